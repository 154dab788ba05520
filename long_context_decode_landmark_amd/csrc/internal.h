// Launchers shared between the kernel translation units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowram {

// Attention workgroups are 4 waves.  Selected chunks: each wave owns
// 16 * kAttSelNT tokens; the exact window: 32 tokens per wave.
#ifndef LOWRAM_ATT_NT
#define LOWRAM_ATT_NT 2
#endif
constexpr int kAttWaves = 4;
constexpr int kAttSelNT = LOWRAM_ATT_NT;
constexpr int kAttChunksWG = kAttWaves * 16 * kAttSelNT / 8;  // selected chunks per workgroup
constexpr int kAttTokWave = 32;                              // window tokens per wave
constexpr int kAttTokWG = kAttWaves * kAttTokWave;           // window tokens per workgroup
constexpr int kPartStride = 2 + 128;                       // m, l, o[128] per query head
constexpr int kMergeMaxSplits = 4096;                      // partial slots per head the merge takes
constexpr int kPipeSplitsPerGroup = 4;                     // producer/consumer kernel: partial slots per group of tiles

// Division by a runtime divisor d >= 1 without a divide loop, for
// 0 <= x < 2^31: q = (mulhi(x, m) + x) >> s with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1 (the round-up method of Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDiv {
  uint32_t m;
  int s, d;
};
inline FastDiv make_fastdiv(int d) {
  FastDiv f{0u, 0, d < 1 ? 1 : d};
  while ((1ll << f.s) < f.d) ++f.s;
  f.m = (uint32_t)((((1ull << 32) * ((1ull << f.s) - (unsigned long long)f.d)) / (unsigned long long)f.d) + 1ull);
  return f;
}
__device__ __forceinline__ int fdiv(int x, const FastDiv& f) {
  return (int)(((unsigned long long)__umulhi((uint32_t)x, f.m) + (uint32_t)x) >> f.s);
}

struct AttendArgs {
  const void* coeff;
  const uint16_t* coeff_scale;
  const uint16_t* basis;
  const uint16_t* w1;
  const uint16_t* b1;
  const uint16_t* w2;
  const uint16_t* b2;
  const int32_t* res_idx;
  const void* res_val;
  const uint16_t* res_scale;
  const uint32_t* res_desc;
  const uint16_t* win_k;
  const uint16_t* win_v;
  const uint16_t* q;
  const int32_t* sel;
  float* part;
  // producer/consumer kernel: PH rows [head][n_ph][g][kHidden] beside the
  // output-space partials of its slots (group gx of a head at row 4 gx)
  float* ph;
  int n_ph;
  float* kpre_out;
  float* kpost_out;
  float* vhat_out;
  int nb, hq, hkv, g, prefix, window, n_chunks, k_eff, n_resid;
  int cache_bmul;  // 1: cache arrays per sequence; 0: one context shared by all nb queries
  int prefix_cap;  // coefficient rows per sequence (descriptor rows per head = prefix_cap / S)
  int window_cap;  // window rows per head
  // partial slots per head: n_split.  The 4-wave kernel treats slots below
  // n_sel_tiles as selection tiles and the rest as window tiles; one launch of
  // it covers slots [split_base, split_base + n_split_launch) of every head
  // (total = heads * n_split_launch workgroups, padded to a multiple of 8).
  int n_sel_tiles, n_win_tiles, n_split, total, padded_total;
  int split_base, n_split_launch;
  // producer/consumer kernel: the pipe_tiles selection tiles of a head are
  // cut into pipe_grp groups of pipe_tpw consecutive tiles (the last may be
  // shorter); group g = head * pipe_grp + gx of the pipe_groups goes to
  // workgroup g % pipe_wgs (grid padded to pipe_padded), and its 4 slots'
  // partials to partial slots 4 gx .. 4 gx + 3 of the head
  int pipe_tiles, pipe_grp, pipe_tpw, pipe_groups, pipe_wgs, pipe_padded;
  FastDiv grp_div, hkv_div;  // by pipe_grp and by hkv
  float scale_log2;
  double inv_freq[64];
};

// Plan of the producer/consumer attention kernel: workgroups (one per CU at
// most), tiles per group, groups per head.
void plan_pipe(int heads, int n_tiles, int n_cu, int* n_wg, int* tpw, int* n_grp);
hipError_t launch_attend_pipe(const AttendArgs& a, int rank, bool coeff_int4, bool resid_int4,
                              hipStream_t st);

// The exact window's tiles when they run as extra workgroups of the score
// grid: n_tiles 128-token tiles per (sequence, KV head), tile i written to
// partial slot slot0 + i of part [head][n_split][g][kPartStride]; window
// rows [cache head][window_cap][d] (cache head as for the landmarks).
struct ScoreWindow {
  const uint16_t* win_k = nullptr;
  const uint16_t* win_v = nullptr;
  float* part = nullptr;
  int n_tiles = 0, window = 0, window_cap = 0, n_split = 0, slot0 = 0;
  float scale_log2 = 0.f;
};
// cache_bmul: 1 = landmarks / candidate ids per sequence, 0 = one shared context
// lm_rows: landmark rows per (sequence, KV head) (>= n_cand)
// win: window tiles to run in the same grid (per-sequence caches only), or none
hipError_t launch_score(const uint16_t* q, const uint16_t* landmark, uint32_t* keys,
                        float* scores_out, int nb, int n_cand, int hq, int hkv, hipStream_t st,
                        int cache_bmul = 1, int lm_rows = -1, const ScoreWindow& win = ScoreWindow{});
hipError_t launch_select(const uint32_t* keys, const int32_t* cand_ids, int32_t* sel,
                         int32_t* sel_out, int nb, int n_cand, int k, int hkv, hipStream_t st,
                         int cache_bmul = 1);
hipError_t launch_attend(const AttendArgs& a, int rank, bool coeff_int4, bool resid_int4,
                         hipStream_t st);
// Exact top-k of n_lists long lists (keys [n_lists][n] -> sel [n_lists][k]
// ascending indices, ties to the lower index), spread over many workgroups;
// ws of split_select_ws_bytes bytes.
size_t split_select_ws_bytes(int n_lists, int n);
hipError_t launch_select_split(const uint32_t* keys, int32_t* sel, int n_lists, int n, int k, void* ws,
                               hipStream_t st, int sel_stride = -1, float* thresh = nullptr);
// Merge of the split partials of every (sequence, KV head, query head).  With
// ph: its first n_ph_used slots form groups of 4, each with one PH row (row
// 4 gx of ph [head][ph_stride][g][kHidden], relative to the largest of the
// group's slot maxima), to which W2 of the head (w2 [cache head][d][kHidden],
// cache head = sequence * cache_bmul * hkv + KV head) is applied.
struct MergePH {
  const float* ph = nullptr;
  int n_ph_used = 0, ph_stride = 0, cache_bmul = 1;
  const uint16_t* w2 = nullptr;
};
hipError_t launch_merge(const float* part, uint16_t* out, int nb, int hkv, int g, int n_split,
                        hipStream_t st, const MergePH& phm = MergePH{});
hipError_t launch_dense(const uint16_t* k, const uint16_t* v, const uint16_t* q, float* part,
                        int nb, int ctx, int hq, int hkv, int n_split, int tok_per_split,
                        float scale_log2, hipStream_t st);
hipError_t launch_chunk_desc(const int32_t* res_idx, int n_lists, int n_resid, int n_chunks,
                             int chunk, uint32_t* desc, hipStream_t st, int idx_stride = -1,
                             int desc_stride = -1);

// Cache builder.
struct BuildGeo {
  int nb, T, P, W, D, r, hkv, layer_in_group, n_chunks, n_resid;
  int prefix_cap, window_cap, resid_cap;  // output strides (coefficient rows, window rows, residual rows)
  double inv_freq[64];
};

// coefficient rows of token t of sequence b go to row b * out_rows + row0 + t
hipError_t launch_proj(const uint16_t* keys, const uint16_t* basis, void* coeff, uint16_t* scale, int nb,
                       int T, int P, int D, int r, bool int4, hipStream_t st, int out_rows = -1,
                       int row0 = 0);
hipError_t launch_build_layer_arrays(const uint16_t* keys, const uint16_t* values, const uint16_t* basis,
                                     uint16_t* blk, uint16_t* lm, uint16_t* wk, uint16_t* wv,
                                     const BuildGeo& g, hipStream_t st);
hipError_t launch_predict_resid(const void* coeff, const uint16_t* coeff_scale, const uint16_t* blk,
                                const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, const uint16_t* b2,
                                const uint16_t* values, float* r, uint32_t* keys, bool ci4, const BuildGeo& g,
                                hipStream_t st);
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st);
hipError_t launch_gemm_nt(const uint16_t* A, const uint16_t* B, int nb, int T, int rows, int K, int r, int mode,
                          float* out_f32, uint16_t* out_t, int ld_t, hipStream_t st, int splits = 1,
                          float* partials = nullptr);
hipError_t launch_fit_basis(const uint16_t* keys, const uint16_t* omega_t, uint16_t* basis_out, int nb, int T,
                            int P, int D, int r, int power, void* ws, int* status, hipStream_t st);
size_t fit_basis_ws_bytes(int P, int D, int r);
struct AppendArgs {
  const uint16_t* keys_new;     // [NB][S][D] pre-RoPE keys of the S tokens
  const void* coeff;            // group coefficients, rows b * prefix_cap + t
  const uint16_t* coeff_scale;
  const uint16_t* blk;          // [NB][Hkv][d][r]
  const uint16_t *w1, *b1, *w2, *b2;
  const float* thresh;          // [NB][Hkv]
  uint16_t* landmark;           // [NB][Hkv][prefix_cap / S][d]
  int32_t* res_idx;             // [NB][Hkv][resid_cap]
  void* res_val;
  uint16_t* res_scale;
  uint32_t* desc;               // [NB][Hkv][prefix_cap / S]
  int32_t* count;               // [NB][Hkv]
  int32_t* dropped;             // [NB][Hkv]
  uint16_t* win_k;              // [NB][Hkv][window_cap][d]
  uint16_t* win_v;
  int D, r, hkv, layer_in_group, P, W, prefix_cap, window_cap, resid_cap;
  bool ci4, ri4;
  double inv_freq[64];
};
hipError_t launch_append(const AppendArgs& a, int nb, hipStream_t st);
hipError_t launch_resid_store(const float* r, const int32_t* idx, void* res_val, uint16_t* res_scale,
                              const BuildGeo& g, bool int4, hipStream_t st);

}  // namespace lowram

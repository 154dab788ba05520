// C ABI of the LowRAM decode-step library: argument checks (before any HIP
// call), workspace carving, and the launch sequence
//   score (landmark GEMV) -> select (exact top-k) -> attend (fused rebuild +
//   split-K attention, window included) -> merge (log-sum-exp of the splits).
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/lowram.h"
#include "common.h"
#include "internal.h"

namespace {

using namespace lowram;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

bool misaligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

// Workgroups of a 1-D grid of 256-thread workgroups: a dispatch counts its
// work-items (workgroups x 256) in 32 bits, and the launches pad the grid to
// a multiple of 8 workgroups, so the limit is the largest multiple of 8 below
// (2^32 - 1) / 256.
constexpr int64_t kMaxGrid1D = ((int64_t)0xFFFFFFFF / 256) & ~(int64_t)7;
// The merge: one 512-thread workgroup per (sequence, query head), also a
// 1-D grid padded to a multiple of 8.
constexpr int64_t kMaxMergeGrid = ((int64_t)0xFFFFFFFF / 512) & ~(int64_t)7;

struct Plan {
  // n_split: partial slots per head of the 4-wave kernel (one per tile);
  // n_part: slots reserved per head, enough for either attention kernel;
  // n_ph: PH rows reserved per head (the producer/consumer kernel's slots)
  int g, n_chunks, n_cand, k_eff, n_sel_tiles, n_win_tiles, n_split, n_part, n_ph;
  size_t off_keys, off_sel, off_part, off_ph, total;
};

int check_shape(const lowram_shape* s) {
  if (!s) return LOWRAM_ERR_NULL;
  if (s->batch < 1 || s->prefix_len < 0 || s->window < 0 || s->n_heads_q < 1 ||
      s->n_heads_kv < 1 || s->topk < 1 || s->n_resid < 0 || s->chunk < 1 || s->head_dim < 1 ||
      s->rank < 1 || s->mlp_hidden < 1)
    return LOWRAM_ERR_SHAPE;
  if (s->n_heads_q % s->n_heads_kv) return LOWRAM_ERR_SHAPE;
  if (s->prefix_len % s->chunk) return LOWRAM_ERR_SHAPE;
  if (s->prefix_len + s->window < 1) return LOWRAM_ERR_SHAPE;
  if (s->n_resid > s->prefix_len) return LOWRAM_ERR_SHAPE;
  if (s->n_resid >= (1 << 24)) return LOWRAM_ERR_UNSUPPORTED;  // 24-bit row field of the descriptor
  if (s->coeff_fmt != LOWRAM_FMT_BF16 && s->coeff_fmt != LOWRAM_FMT_INT4_G32) return LOWRAM_ERR_SHAPE;
  if (s->resid_fmt != LOWRAM_FMT_BF16 && s->resid_fmt != LOWRAM_FMT_INT4_G32) return LOWRAM_ERR_SHAPE;
  if (!(s->rope_theta > 0.f) || !std::isfinite(s->rope_theta)) return LOWRAM_ERR_SHAPE;
  if (!std::isfinite(s->softmax_scale)) return LOWRAM_ERR_SHAPE;
  const int n_chunks = s->prefix_len / s->chunk;
  if (s->n_cand < 0 || s->n_cand > n_chunks) return LOWRAM_ERR_SHAPE;
  if (s->chunk != kChunk || s->head_dim != kHeadDim || s->mlp_hidden != kHidden)
    return LOWRAM_ERR_UNSUPPORTED;
  if (s->n_heads_q / s->n_heads_kv > 16) return LOWRAM_ERR_UNSUPPORTED;
  if (s->rank != 64 && s->rank != 128 && s->rank != 256 && s->rank != 512) return LOWRAM_ERR_UNSUPPORTED;
  if (s->coeff_fmt == LOWRAM_FMT_INT4_G32 && s->rank % 128) return LOWRAM_ERR_UNSUPPORTED;
  if (s->prefix_cap < 0 || s->window_cap < 0) return LOWRAM_ERR_SHAPE;
  if (s->prefix_cap && (s->prefix_cap < s->prefix_len || s->prefix_cap % s->chunk)) return LOWRAM_ERR_SHAPE;
  if (s->window_cap && s->window_cap < s->window) return LOWRAM_ERR_SHAPE;
  // 32-bit index arithmetic inside the kernels
  if ((int64_t)s->batch * (s->prefix_cap ? s->prefix_cap : s->prefix_len) >= (int64_t)1 << 31)
    return LOWRAM_ERR_UNSUPPORTED;
  // grid limits: sequences and KV heads index the y and z grid dimensions
  // (at most 65535), and the 4-wave grid has one workgroup per (sequence,
  // KV head, tile)
  if (s->batch > 65535 || s->n_heads_kv > 65535) return LOWRAM_ERR_UNSUPPORTED;
  const int64_t k_eff = s->n_cand < s->topk ? s->n_cand : s->topk;
  const int64_t tiles = (k_eff + kAttChunksWG - 1) / kAttChunksWG + (s->window + kAttTokWG - 1) / kAttTokWG;
  if ((int64_t)s->batch * s->n_heads_kv * tiles > kMaxGrid1D) return LOWRAM_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->n_heads_q > kMaxMergeGrid) return LOWRAM_ERR_UNSUPPORTED;
  // nothing to attend: no candidate chunk and no window token gives no split
  if (s->n_cand == 0 && s->window == 0) return LOWRAM_ERR_SHAPE;
  return LOWRAM_OK;
}

int prefix_rows(const lowram_shape* s) { return s->prefix_cap ? s->prefix_cap : s->prefix_len; }
int window_rows(const lowram_shape* s) { return s->window_cap ? s->window_cap : s->window; }

// Kernel for the selected chunks: 0 automatic, 1 producer/consumer, 2 four-wave
// (environment variable LOWRAM_ATTEND = pipe | wave; anything else: automatic).
int attend_mode() {
  const char* v = std::getenv("LOWRAM_ATTEND");
  if (!v) return 0;
  if (std::strcmp(v, "pipe") == 0) return 1;
  if (std::strcmp(v, "wave") == 0) return 2;
  return 0;
}

// CUs to plan the producer/consumer kernel for (environment variable
// LOWRAM_PIPE_CUS = n >= 1); 0: the device's count.
int pipe_cus_override() {
  const char* v = std::getenv("LOWRAM_PIPE_CUS");
  if (!v) return 0;
  const long n = std::strtol(v, nullptr, 10);
  return n >= 1 && n <= 65536 ? (int)n : 0;
}

Plan make_plan(const lowram_shape* s) {
  Plan p{};
  p.g = s->n_heads_q / s->n_heads_kv;
  p.n_chunks = s->prefix_len / s->chunk;
  p.n_cand = s->n_cand;
  p.k_eff = p.n_cand < s->topk ? p.n_cand : s->topk;
  p.n_sel_tiles = (p.k_eff + kAttChunksWG - 1) / kAttChunksWG;
  p.n_win_tiles = (s->window + kAttTokWG - 1) / kAttTokWG;
  p.n_split = p.n_sel_tiles + p.n_win_tiles;
  // The producer/consumer kernel writes 4 slots per group of tiles, and its
  // groups hold at least 2 tiles where a head has 2: 2 n + 6 slots cover it.
  p.n_ph = p.n_sel_tiles > 0 ? 2 * p.n_sel_tiles + 6 : 0;
  p.n_part = p.n_ph + p.n_win_tiles;
  const size_t heads = (size_t)s->batch * s->n_heads_kv;
  p.off_keys = 0;
  p.off_sel = align_up(heads * (size_t)p.n_cand * 4);
  p.off_part = p.off_sel + align_up(heads * (size_t)p.k_eff * 4);
  p.off_ph = p.off_part + align_up(heads * (size_t)p.n_part * p.g * kPartStride * 4);
  p.total = p.off_ph + align_up(heads * (size_t)p.n_ph * p.g * kHidden * 4);
  return p;
}

// Which kernel runs the selected chunks, and the producer/consumer kernel's
// plan.  mode: 0 automatic, 1 producer/consumer forced, 2 4-wave forced.
struct AttendPlan {
  bool pipe;
  int n_wg, tpw, n_grp, sel_slots, n_split;
};
AttendPlan attend_plan(const lowram_shape* s, const Plan& p, bool stage_outputs, int n_cu, int mode) {
  // The producer/consumer kernel: one workgroup per CU working through
  // groups of tiles, 4 partial slots per group.  It pays off once every CU
  // gets more than 2 tiles (its pipeline fills and drains once per workgroup,
  // and its merge applies W2; at 2 tiles per CU the 4-wave kernel measured
  // faster);
  // small problems, every call that asks for stage outputs, and shapes whose
  // partial slots would not fit the reserve or the merge run the 4-wave
  // kernel (one slot per tile).  A forced mode overrides the size rule only.
  // The exact window always goes to the 4-wave kernel, in the slots after
  // the selection's.
  const bool has_prefix = s->prefix_len > 0 && p.n_cand > 0;
  const int heads = s->batch * s->n_heads_kv;
  AttendPlan a{false, 0, 0, 0, 0, 0};
  if (has_prefix) plan_pipe(heads, p.n_sel_tiles, n_cu, &a.n_wg, &a.tpw, &a.n_grp);
  const long long all_tiles = (long long)heads * p.n_sel_tiles;
  const int pipe_split = kPipeSplitsPerGroup * a.n_grp + p.n_win_tiles;
  const bool fits = a.n_wg > 0 && pipe_split <= p.n_part && pipe_split <= kMergeMaxSplits;
  a.pipe = has_prefix && !stage_outputs && fits && (mode == 0 ? all_tiles > 2LL * n_cu : mode == 1);
  a.sel_slots = !has_prefix ? 0 : a.pipe ? kPipeSplitsPerGroup * a.n_grp : p.n_sel_tiles;
  a.n_split = a.sel_slots + p.n_win_tiles;
  return a;
}

// Where the exact window's tiles run: as extra workgroups of the score
// launch when the selected chunks go to the producer/consumer kernel and the
// caches are per sequence (it would otherwise take a launch of its own;
// the 4-wave kernel takes the window tiles into its own grid).
bool window_in_score(const lowram_shape* s, const Plan& p, const AttendPlan& ap, bool shared) {
  const bool has_prefix = s->prefix_len > 0 && p.n_cand > 0;
  return has_prefix && ap.pipe && !shared && p.n_win_tiles > 0;
}

// CUs the producer/consumer kernel is planned for: LOWRAM_PIPE_CUS, else the
// current device's count (256 if it cannot be read).
int plan_cus() {
  int n_cu = pipe_cus_override();
  if (n_cu <= 0) {
    n_cu = 256;
    int dev = 0, cu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cu > 0)
      n_cu = cu;
  }
  return n_cu;
}

// Every argument check of a decode step except the workspace's (no HIP call).
int check_step(const lowram_shape* s, const lowram_layer_cache* c, const uint16_t* q, uint16_t* out,
               int32_t* sel_out, float* scores_out, float* kpre_out, float* kpost_out, float* vhat_out) {
  int st = check_shape(s);
  if (st) return st;
  if (!c || !q || !out) return LOWRAM_ERR_NULL;
  const Plan p = make_plan(s);
  const bool has_prefix = s->prefix_len > 0 && p.n_cand > 0;
  const bool ci4 = s->coeff_fmt == LOWRAM_FMT_INT4_G32, ri4 = s->resid_fmt == LOWRAM_FMT_INT4_G32;
  if (has_prefix) {
    if (!c->coeff || !c->basis || !c->landmark || !c->w1 || !c->b1 || !c->w2 || !c->b2 ||
        !c->res_chunk_desc)
      return LOWRAM_ERR_NULL;
    if (s->n_resid > 0 && (!c->res_idx || !c->res_val)) return LOWRAM_ERR_NULL;
    if (ci4 && !c->coeff_scale) return LOWRAM_ERR_NULL;
    if (ri4 && s->n_resid > 0 && !c->res_scale) return LOWRAM_ERR_NULL;
    if (!c->cand_ids && p.n_cand != p.n_chunks) return LOWRAM_ERR_SHAPE;
    if (c->cand_ids && (s->prefix_cap || s->window_cap)) return LOWRAM_ERR_SHAPE;  // eviction: dense only
  }
  if (s->window > 0 && (!c->win_k || !c->win_v)) return LOWRAM_ERR_NULL;
  const void* bulk[] = {q, out, c->coeff, c->basis, c->landmark, c->w1, c->w2, c->res_val,
                        c->win_k, c->win_v};
  for (const void* ptr : bulk)
    if (ptr && misaligned(ptr, 16)) return LOWRAM_ERR_ALIGN;
  const void* small[] = {c->coeff_scale, c->cand_ids, c->b1, c->b2, c->res_idx, c->res_scale,
                         c->res_chunk_desc, sel_out, scores_out, kpre_out, kpost_out, vhat_out};
  for (const void* ptr : small)
    if (ptr && misaligned(ptr, 4)) return LOWRAM_ERR_ALIGN;
  if (kpre_out && misaligned(kpre_out, 16)) return LOWRAM_ERR_ALIGN;
  if (kpost_out && misaligned(kpost_out, 16)) return LOWRAM_ERR_ALIGN;
  if (p.n_split > kMergeMaxSplits) return LOWRAM_ERR_UNSUPPORTED;
  return LOWRAM_OK;
}

// The launches of a decode step whose arguments check_step accepted, with a
// workspace of at least make_plan(s).total bytes.
int launch_step(const lowram_shape* s, const lowram_layer_cache* c, const uint16_t* q, uint16_t* out,
                int32_t* sel_out, float* scores_out, float* kpre_out, float* kpost_out,
                float* vhat_out, void* ws, void* stream, void* const* events, bool shared) {
  const Plan p = make_plan(s);
  const bool has_prefix = s->prefix_len > 0 && p.n_cand > 0;
  const bool ci4 = s->coeff_fmt == LOWRAM_FMT_INT4_G32, ri4 = s->resid_fmt == LOWRAM_FMT_INT4_G32;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  unsigned char* w = static_cast<unsigned char*>(ws);
  uint32_t* keys = reinterpret_cast<uint32_t*>(w + p.off_keys);
  int32_t* sel = reinterpret_cast<int32_t*>(w + p.off_sel);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  float* ph = reinterpret_cast<float*>(w + p.off_ph);
  auto mark = [&](int i) {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[i]), hs) == hipSuccess;
  };

  const int heads = s->batch * s->n_heads_kv;
  const AttendPlan ap = attend_plan(s, p, kpre_out || kpost_out || vhat_out, plan_cus(), attend_mode());
  const bool wave4 = !ap.pipe;
  const int n_split = ap.n_split;
  const float scale_log2 = s->softmax_scale * 1.4426950408889634f;
  const bool win_score = window_in_score(s, p, ap, shared);

  if (!mark(0)) return LOWRAM_ERR_HIP;
  if (has_prefix) {
    ScoreWindow sw;
    if (win_score) {
      sw.win_k = c->win_k; sw.win_v = c->win_v; sw.part = part;
      sw.n_tiles = p.n_win_tiles; sw.window = s->window; sw.window_cap = window_rows(s);
      sw.n_split = n_split; sw.slot0 = ap.sel_slots; sw.scale_log2 = scale_log2;
    }
    if (launch_score(q, c->landmark, keys, scores_out, s->batch, p.n_cand, s->n_heads_q,
                     s->n_heads_kv, hs, shared ? 0 : 1, c->cand_ids ? p.n_cand : prefix_rows(s) / s->chunk,
                     sw) != hipSuccess)
      return LOWRAM_ERR_HIP;
  }
  if (!mark(1)) return LOWRAM_ERR_HIP;
  if (has_prefix || sel_out) {
    if (launch_select(keys, c->cand_ids, sel, sel_out, s->batch, p.n_cand, s->topk, s->n_heads_kv,
                      hs, shared ? 0 : 1) != hipSuccess)
      return LOWRAM_ERR_HIP;
  }
  if (!mark(2)) return LOWRAM_ERR_HIP;
  AttendArgs a{};
  a.coeff = c->coeff; a.coeff_scale = c->coeff_scale; a.basis = c->basis;
  a.w1 = c->w1; a.b1 = c->b1; a.w2 = c->w2; a.b2 = c->b2;
  a.res_idx = c->res_idx; a.res_val = c->res_val; a.res_scale = c->res_scale;
  a.res_desc = c->res_chunk_desc; a.win_k = c->win_k; a.win_v = c->win_v;
  a.q = q; a.sel = sel; a.part = part; a.ph = ph; a.n_ph = p.n_ph;
  a.kpre_out = kpre_out; a.kpost_out = kpost_out; a.vhat_out = vhat_out;
  a.nb = s->batch; a.hq = s->n_heads_q; a.hkv = s->n_heads_kv; a.g = p.g;
  a.prefix = s->prefix_len; a.window = s->window; a.n_chunks = p.n_chunks; a.k_eff = p.k_eff;
  a.n_resid = s->n_resid;
  a.cache_bmul = shared ? 0 : 1;
  a.prefix_cap = prefix_rows(s);
  a.window_cap = window_rows(s);
  a.n_sel_tiles = ap.sel_slots;
  a.n_win_tiles = p.n_win_tiles;
  a.n_split = n_split;
  a.split_base = wave4 ? 0 : ap.sel_slots;
  a.n_split_launch = wave4 ? n_split : p.n_win_tiles;
  // (no launch of its own for the window when the score grid ran it)
  a.total = win_score ? 0 : heads * a.n_split_launch;
  a.padded_total = (a.total + 7) & ~7;
  a.pipe_tiles = p.n_sel_tiles;
  a.pipe_grp = ap.n_grp;
  a.pipe_tpw = ap.tpw;
  a.pipe_groups = wave4 ? 0 : heads * ap.n_grp;
  a.pipe_wgs = wave4 ? 0 : ap.n_wg;
  a.pipe_padded = (a.pipe_wgs + 7) & ~7;
  a.grp_div = make_fastdiv(ap.n_grp);
  a.hkv_div = make_fastdiv(s->n_heads_kv);
  a.scale_log2 = scale_log2;
  for (int i = 0; i < 64; ++i)
    a.inv_freq[i] = std::pow((double)s->rope_theta, -2.0 * i / (double)kHeadDim);
  if (launch_attend(a, s->rank, ci4, ri4, hs) != hipSuccess) return LOWRAM_ERR_HIP;
  if (launch_attend_pipe(a, s->rank, ci4, ri4, hs) != hipSuccess) return LOWRAM_ERR_HIP;
  if (!mark(3)) return LOWRAM_ERR_HIP;
  MergePH phm;
  if (ap.pipe) {  // the producer/consumer kernel's slots leave W2 to the merge
    phm.ph = ph;
    phm.n_ph_used = ap.sel_slots;
    phm.ph_stride = p.n_ph;
    phm.cache_bmul = a.cache_bmul;
    phm.w2 = c->w2;
  }
  if (launch_merge(part, out, s->batch, s->n_heads_kv, p.g, n_split, hs, phm) != hipSuccess)
    return LOWRAM_ERR_HIP;
  if (!mark(4)) return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}

int run_step(const lowram_shape* s, const lowram_layer_cache* c, const uint16_t* q, uint16_t* out,
             int32_t* sel_out, float* scores_out, float* kpre_out, float* kpost_out,
             float* vhat_out, void* ws, size_t ws_bytes, void* stream,
             void* const* events = nullptr, bool shared = false) {
  const int st = check_step(s, c, q, out, sel_out, scores_out, kpre_out, kpost_out, vhat_out);
  if (st) return st;
  if (!ws) return LOWRAM_ERR_NULL;
  if (misaligned(ws, 16)) return LOWRAM_ERR_ALIGN;
  if (ws_bytes < make_plan(s).total) return LOWRAM_ERR_WORKSPACE;
  return launch_step(s, c, q, out, sel_out, scores_out, kpre_out, kpost_out, vhat_out, ws, stream, events,
                     shared);
}

// ---------------------------------------------------------------------------
// Fixed scratch of the no-allocation decode step.  Each GPU the library runs
// on holds its own copy of this array from the library's load until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[LOWRAM_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (looked up at the first call on
// that device).
int scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LOWRAM_ERR_HIP;
  if (dev < 0 || dev >= kScratchDevices) return LOWRAM_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LOWRAM_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return LOWRAM_OK;
}

constexpr int kDenseTokPerSplit = 2048;
int check_dense(const dense_shape* s) {
  if (!s) return LOWRAM_ERR_NULL;
  if (s->batch < 1 || s->ctx_len < 1 || s->n_heads_q < 1 || s->n_heads_kv < 1 || s->head_dim < 1)
    return LOWRAM_ERR_SHAPE;
  if (s->n_heads_q % s->n_heads_kv) return LOWRAM_ERR_SHAPE;
  if (!std::isfinite(s->softmax_scale)) return LOWRAM_ERR_SHAPE;
  if (s->head_dim != kHeadDim || s->n_heads_q / s->n_heads_kv > 16) return LOWRAM_ERR_UNSUPPORTED;
  // grid limits, as for the decode step
  if (s->batch > 65535 || s->n_heads_kv > 65535) return LOWRAM_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->n_heads_kv * ((s->ctx_len + kDenseTokPerSplit - 1) / kDenseTokPerSplit) >
      kMaxGrid1D)
    return LOWRAM_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->n_heads_q > kMaxMergeGrid) return LOWRAM_ERR_UNSUPPORTED;
  return LOWRAM_OK;
}

int check_build_shape(const lowram_build_shape* s) {
  if (!s) return LOWRAM_ERR_NULL;
  if (s->batch < 1 || s->ctx_len < 1 || s->window < 0 || s->window > s->ctx_len || s->chunk < 1 ||
      s->n_heads_kv < 1 || s->head_dim < 1 || s->rank < 1 || s->group_layers < 1 || s->mlp_hidden < 1 ||
      s->n_resid < 0)
    return LOWRAM_ERR_SHAPE;
  const int P = s->ctx_len - s->window;
  if (P % s->chunk) return LOWRAM_ERR_SHAPE;
  if (s->n_resid > P) return LOWRAM_ERR_SHAPE;
  if (s->coeff_fmt != LOWRAM_FMT_BF16 && s->coeff_fmt != LOWRAM_FMT_INT4_G32) return LOWRAM_ERR_SHAPE;
  if (s->resid_fmt != LOWRAM_FMT_BF16 && s->resid_fmt != LOWRAM_FMT_INT4_G32) return LOWRAM_ERR_SHAPE;
  if (!(s->rope_theta > 0.f) || !std::isfinite(s->rope_theta)) return LOWRAM_ERR_SHAPE;
  if (s->chunk != kChunk || s->head_dim != kHeadDim || s->mlp_hidden != kHidden) return LOWRAM_ERR_UNSUPPORTED;
  if (s->rank != 64 && s->rank != 128 && s->rank != 256 && s->rank != 512) return LOWRAM_ERR_UNSUPPORTED;
  if (s->coeff_fmt == LOWRAM_FMT_INT4_G32 && s->rank % 128) return LOWRAM_ERR_UNSUPPORTED;
  if (s->n_resid >= (1 << 24)) return LOWRAM_ERR_UNSUPPORTED;
  if (s->prefix_cap < 0 || s->window_cap < 0 || s->resid_cap < 0) return LOWRAM_ERR_SHAPE;
  if (s->prefix_cap && (s->prefix_cap < P || s->prefix_cap % s->chunk)) return LOWRAM_ERR_SHAPE;
  if (s->window_cap && s->window_cap < s->window) return LOWRAM_ERR_SHAPE;
  if (s->resid_cap && s->resid_cap < s->n_resid) return LOWRAM_ERR_SHAPE;
  if (s->resid_cap >= (1 << 24)) return LOWRAM_ERR_UNSUPPORTED;
  // 32-bit token and element indices inside the kernels
  if ((int64_t)s->batch * s->ctx_len >= (int64_t)1 << 31) return LOWRAM_ERR_UNSUPPORTED;
  if ((int64_t)s->batch * s->prefix_cap >= (int64_t)1 << 31) return LOWRAM_ERR_UNSUPPORTED;
  if ((int64_t)s->group_layers * s->n_heads_kv * kHeadDim >= (int64_t)1 << 20) return LOWRAM_ERR_UNSUPPORTED;
  if (s->batch > 65535) return LOWRAM_ERR_UNSUPPORTED;  // a grid dimension of at most 65535
  // the residual top-k and descriptor grids index (sequence, KV head) lists
  // in a grid dimension of at most 65535
  if ((int64_t)s->batch * s->n_heads_kv > 65535) return LOWRAM_ERR_UNSUPPORTED;
  // 1-D grids of 256-thread workgroups: the projection (128-token tiles x
  // 128-column blocks of the rank) and the residual prediction (128-token
  // tiles per (sequence, KV head))
  const int64_t tok_tiles = (P + 127) / 128;
  if ((int64_t)s->batch * tok_tiles * ((s->rank + 127) / 128) > kMaxGrid1D ||
      (int64_t)s->batch * s->n_heads_kv * tok_tiles > kMaxGrid1D)
    return LOWRAM_ERR_UNSUPPORTED;
  return LOWRAM_OK;
}

struct BuildPlan {
  int P, n_chunks;
  size_t off_r, off_keys, off_sel, total;
};

BuildPlan make_build_plan(const lowram_build_shape* s) {
  BuildPlan p{};
  p.P = s->ctx_len - s->window;
  p.n_chunks = p.P / s->chunk;
  const size_t heads = (size_t)s->batch * s->n_heads_kv;
  p.off_r = 0;                                                // fp32 residual rows [NB][Hkv][P][d]
  p.off_keys = align_up(heads * (size_t)p.P * kHeadDim * 4);  // uint32 error keys [NB][Hkv][P]
  p.off_sel = p.off_keys + align_up(heads * (size_t)p.P * 4);  // top-k histograms and counts
  p.total = p.off_sel + (p.P > 0 ? align_up(split_select_ws_bytes((int)heads, p.P)) : 0);
  return p;
}


int dense_splits(const dense_shape* s) { return (s->ctx_len + kDenseTokPerSplit - 1) / kDenseTokPerSplit; }

}  // namespace

extern "C" {

int lowram_abi_version(void) { return LOWRAM_ABI_VERSION; }

const char* lowram_strerror(int status) {
  switch (status) {
    case LOWRAM_OK: return "ok";
    case LOWRAM_ERR_NULL: return "a required pointer is NULL";
    case LOWRAM_ERR_SHAPE: return "inconsistent shape";
    case LOWRAM_ERR_UNSUPPORTED: return "shape not supported by this library";
    case LOWRAM_ERR_WORKSPACE: return "workspace too small";
    case LOWRAM_ERR_ALIGN: return "misaligned pointer";
    case LOWRAM_ERR_HIP: return "HIP launch failed";
    case LOWRAM_ERR_SCRATCH:
      return "the shape needs more workspace than the fixed no-allocation scratch holds "
             "(LOWRAM_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int lowram_workspace_bytes(const lowram_shape* shape, size_t* bytes) {
  if (!bytes) return LOWRAM_ERR_NULL;
  const int st = check_shape(shape);
  if (st) return st;
  *bytes = make_plan(shape).total;
  return LOWRAM_OK;
}

int lowram_decode_plan(const lowram_shape* shape, int n_cu, int mode, lowram_attend_plan* plan) {
  if (!plan) return LOWRAM_ERR_NULL;
  const int st = check_shape(shape);
  if (st) return st;
  if (n_cu < 1 || mode < 0 || mode > 2) return LOWRAM_ERR_SHAPE;
  const Plan p = make_plan(shape);
  const AttendPlan a = attend_plan(shape, p, false, n_cu, mode);
  const bool has_prefix = shape->prefix_len > 0 && p.n_cand > 0;
  plan->kernel = !has_prefix ? 0 : a.pipe ? 1 : 2;
  plan->workgroups = a.pipe ? a.n_wg : 0;
  plan->tiles_per_group = a.pipe ? a.tpw : 0;
  plan->groups_per_head = a.pipe ? a.n_grp : 0;
  plan->partial_slots = a.n_split;
  plan->reserved_slots = p.n_part;
  plan->window_kernel = p.n_win_tiles == 0 ? 0 : window_in_score(shape, p, a, false) ? 1 : 2;
  return LOWRAM_OK;
}

int lowram_decode_step(const lowram_shape* shape, const lowram_layer_cache* cache,
                       const uint16_t* q, uint16_t* out, int32_t* sel_out, void* workspace,
                       size_t ws_bytes, void* stream) {
  return run_step(shape, cache, q, out, sel_out, nullptr, nullptr, nullptr, nullptr, workspace,
                  ws_bytes, stream);
}

int lowram_decode_step_noalloc(const lowram_shape* shape, const lowram_layer_cache* cache,
                               const uint16_t* q, uint16_t* out, int32_t* sel_out, void* stream) {
  const int st = check_step(shape, cache, q, out, sel_out, nullptr, nullptr, nullptr, nullptr);
  if (st) return st;
  if (make_plan(shape).total > (size_t)LOWRAM_NOALLOC_SCRATCH_BYTES) return LOWRAM_ERR_SCRATCH;
  void* ws = nullptr;
  const int sp = scratch_ptr(&ws);
  if (sp) return sp;
  return launch_step(shape, cache, q, out, sel_out, nullptr, nullptr, nullptr, nullptr, ws, stream, nullptr,
                     false);
}

int lowram_decode_step_events(const lowram_shape* shape, const lowram_layer_cache* cache,
                              const uint16_t* q, uint16_t* out, int32_t* sel_out, void* workspace,
                              size_t ws_bytes, void* stream, void* const* events) {
  return run_step(shape, cache, q, out, sel_out, nullptr, nullptr, nullptr, nullptr, workspace,
                  ws_bytes, stream, events);
}

int lowram_decode_shared(const lowram_shape* shape, const lowram_layer_cache* cache, const uint16_t* q,
                         uint16_t* out, int32_t* sel_out, void* workspace, size_t ws_bytes, void* stream,
                         void* const* events) {
  return run_step(shape, cache, q, out, sel_out, nullptr, nullptr, nullptr, nullptr, workspace, ws_bytes,
                  stream, events, true);
}

int lowram_decode_stages(const lowram_shape* shape, const lowram_layer_cache* cache,
                         const uint16_t* q, uint16_t* out, int32_t* sel_out, float* scores_out,
                         float* kpre_out, float* kpost_out, float* vhat_out, void* workspace,
                         size_t ws_bytes, void* stream) {
  return run_step(shape, cache, q, out, sel_out, scores_out, kpre_out, kpost_out, vhat_out,
                  workspace, ws_bytes, stream);
}

int dense_workspace_bytes(const dense_shape* shape, size_t* bytes) {
  if (!bytes) return LOWRAM_ERR_NULL;
  const int st = check_dense(shape);
  if (st) return st;
  *bytes = align_up((size_t)shape->batch * shape->n_heads_q * dense_splits(shape) * kPartStride * 4);
  return LOWRAM_OK;
}

int dense_decode_step(const dense_shape* shape, const dense_layer_cache* cache, const uint16_t* q,
                      uint16_t* out, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_dense(shape);
  if (st) return st;
  if (!cache || !cache->k || !cache->v || !q || !out || !workspace) return LOWRAM_ERR_NULL;
  const void* bulk[] = {cache->k, cache->v, q, out, workspace};
  for (const void* ptr : bulk)
    if (misaligned(ptr, 16)) return LOWRAM_ERR_ALIGN;
  size_t need = 0;
  dense_workspace_bytes(shape, &need);
  if (dense_splits(shape) > kMergeMaxSplits)
    return LOWRAM_ERR_UNSUPPORTED;
  if (ws_bytes < need) return LOWRAM_ERR_WORKSPACE;
  const int n_split = dense_splits(shape);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float* part = static_cast<float*>(workspace);
  if (launch_dense(cache->k, cache->v, q, part, shape->batch, shape->ctx_len, shape->n_heads_q,
                   shape->n_heads_kv, n_split, kDenseTokPerSplit,
                   shape->softmax_scale * 1.4426950408889634f, hs) != hipSuccess)
    return LOWRAM_ERR_HIP;
  if (launch_merge(part, out, shape->batch, shape->n_heads_kv, shape->n_heads_q / shape->n_heads_kv,
                   n_split, hs) != hipSuccess)
    return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}

int lowram_resid_chunk_desc(const int32_t* res_idx, int32_t n_lists, int32_t n_resid,
                            int32_t n_chunks, int32_t chunk, uint32_t* desc, void* stream) {
  if (!desc || (n_resid > 0 && !res_idx)) return LOWRAM_ERR_NULL;
  if (n_lists < 0 || n_resid < 0 || n_chunks < 0 || chunk < 1) return LOWRAM_ERR_SHAPE;
  if (chunk > 8 || n_resid >= (1 << 24)) return LOWRAM_ERR_UNSUPPORTED;
  if (n_lists > 65535) return LOWRAM_ERR_UNSUPPORTED;  // lists index a grid dimension of at most 65535
  if (misaligned(desc, 4) || (res_idx && misaligned(res_idx, 4))) return LOWRAM_ERR_ALIGN;
  if (n_lists == 0 || n_chunks == 0) return LOWRAM_OK;
  if (launch_chunk_desc(res_idx, n_lists, n_resid, n_chunks, chunk, desc,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
    return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}


int lowram_build_coeff(const lowram_build_shape* shape, const uint16_t* keys, const uint16_t* basis,
                       void* coeff, uint16_t* coeff_scale, void* stream) {
  const int st = check_build_shape(shape);
  if (st) return st;
  const bool ci4 = shape->coeff_fmt == LOWRAM_FMT_INT4_G32;
  const int P = shape->ctx_len - shape->window;
  if (P == 0) return LOWRAM_OK;  // nothing to project
  if (!keys || !basis || !coeff || (ci4 && !coeff_scale)) return LOWRAM_ERR_NULL;
  if (misaligned(keys, 16) || misaligned(basis, 16) || misaligned(coeff, 16) ||
      (coeff_scale && misaligned(coeff_scale, 4)))
    return LOWRAM_ERR_ALIGN;
  const int D = shape->group_layers * shape->n_heads_kv * kHeadDim;
  if (launch_proj(keys, basis, coeff, coeff_scale, shape->batch, shape->ctx_len, P, D, shape->rank, ci4,
                  static_cast<hipStream_t>(stream), shape->prefix_cap ? shape->prefix_cap : P) != hipSuccess)
    return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}

int lowram_build_layer_workspace_bytes(const lowram_build_shape* shape, size_t* bytes) {
  if (!bytes) return LOWRAM_ERR_NULL;
  const int st = check_build_shape(shape);
  if (st) return st;
  *bytes = make_build_plan(shape).total;
  return LOWRAM_OK;
}

namespace {
int run_build_layer(const lowram_build_shape* s, int32_t layer_in_group, const lowram_layer_build* io,
                    void* workspace, size_t ws_bytes, void* stream, void* const* events) {
  int st = check_build_shape(s);
  if (st) return st;
  if (layer_in_group < 0 || layer_in_group >= s->group_layers) return LOWRAM_ERR_SHAPE;
  const BuildPlan p = make_build_plan(s);
  if (!io || (!workspace && p.total > 0)) return LOWRAM_ERR_NULL;  // no prefix: no workspace needed
  const bool ci4 = s->coeff_fmt == LOWRAM_FMT_INT4_G32, ri4 = s->resid_fmt == LOWRAM_FMT_INT4_G32;
  if (!io->keys || !io->group_basis || !io->basis) return LOWRAM_ERR_NULL;
  if (p.P > 0) {
    if (!io->coeff || !io->w1 || !io->b1 || !io->w2 || !io->b2 || !io->landmark || !io->res_chunk_desc)
      return LOWRAM_ERR_NULL;
    if (ci4 && !io->coeff_scale) return LOWRAM_ERR_NULL;
    if (s->n_resid > 0 && (!io->res_idx || !io->res_val || (ri4 && !io->res_scale))) return LOWRAM_ERR_NULL;
  }
  if (s->window > 0 && (!io->values || !io->win_k || !io->win_v)) return LOWRAM_ERR_NULL;
  if (p.P > 0 && s->n_resid > 0 && !io->values) return LOWRAM_ERR_NULL;
  const void* bulk[] = {workspace, io->keys, io->group_basis, io->coeff, io->values, io->w1, io->w2,
                        io->basis, io->landmark, io->res_val, io->win_k, io->win_v};
  for (const void* ptr : bulk)
    if (ptr && misaligned(ptr, 16)) return LOWRAM_ERR_ALIGN;
  const void* small[] = {io->coeff_scale, io->b1,      io->b2,         io->res_idx,
                         io->res_scale,   io->res_chunk_desc, io->res_thresh, io->res_count};
  for (const void* ptr : small)
    if (ptr && misaligned(ptr, 4)) return LOWRAM_ERR_ALIGN;
  if (ws_bytes < p.total) return LOWRAM_ERR_WORKSPACE;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) {
    return !events || hipEventRecord(static_cast<hipEvent_t>(events[i]), hs) == hipSuccess;
  };
  BuildGeo g{};
  g.nb = s->batch; g.T = s->ctx_len; g.P = p.P; g.W = s->window;
  g.D = s->group_layers * s->n_heads_kv * kHeadDim; g.r = s->rank; g.hkv = s->n_heads_kv;
  g.layer_in_group = layer_in_group; g.n_chunks = p.n_chunks; g.n_resid = s->n_resid;
  g.prefix_cap = s->prefix_cap ? s->prefix_cap : p.P;
  g.window_cap = s->window_cap ? s->window_cap : s->window;
  g.resid_cap = s->resid_cap ? s->resid_cap : s->n_resid;
  for (int i = 0; i < 64; ++i) g.inv_freq[i] = std::pow((double)s->rope_theta, -2.0 * i / (double)kHeadDim);
  if (!mark(0)) return LOWRAM_ERR_HIP;
  if (launch_build_layer_arrays(io->keys, io->values, io->group_basis, io->basis, io->landmark, io->win_k,
                                io->win_v, g, hs) != hipSuccess)
    return LOWRAM_ERR_HIP;
  if (!mark(1)) return LOWRAM_ERR_HIP;
  if (p.P == 0) {
    const int heads0 = s->batch * s->n_heads_kv;
    if (io->res_thresh && launch_select_split(nullptr, nullptr, heads0, 0, 0, nullptr, hs, 0, io->res_thresh) !=
                              hipSuccess)
      return LOWRAM_ERR_HIP;  // threshold +inf: no residuals
    if (io->res_count && launch_fill_i32(io->res_count, heads0, 0, hs) != hipSuccess) return LOWRAM_ERR_HIP;
    return mark(2) && mark(3) && mark(4) ? LOWRAM_OK : LOWRAM_ERR_HIP;
  }

  unsigned char* w = static_cast<unsigned char*>(workspace);
  float* r = reinterpret_cast<float*>(w + p.off_r);
  uint32_t* keys = reinterpret_cast<uint32_t*>(w + p.off_keys);
  const size_t heads = (size_t)s->batch * s->n_heads_kv;
  if (s->n_resid > 0) {
    if (launch_predict_resid(io->coeff, io->coeff_scale, io->basis, io->w1, io->b1, io->w2, io->b2, io->values, r,
                             keys, ci4, g, hs) != hipSuccess)
      return LOWRAM_ERR_HIP;
  }
  if (!mark(2)) return LOWRAM_ERR_HIP;
  if (s->n_resid > 0 || io->res_thresh) {
    if (launch_select_split(keys, io->res_idx, (int)heads, p.P, s->n_resid, w + p.off_sel, hs, g.resid_cap,
                            io->res_thresh) != hipSuccess)
      return LOWRAM_ERR_HIP;
  }
  if (io->res_count && launch_fill_i32(io->res_count, (int)heads, s->n_resid, hs) != hipSuccess)
    return LOWRAM_ERR_HIP;
  if (!mark(3)) return LOWRAM_ERR_HIP;
  if (s->n_resid > 0) {
    if (launch_resid_store(r, io->res_idx, io->res_val, io->res_scale, g, ri4, hs) != hipSuccess)
      return LOWRAM_ERR_HIP;
  }
  if (launch_chunk_desc(io->res_idx, (int)heads, s->n_resid, p.n_chunks, s->chunk, io->res_chunk_desc, hs,
                        g.resid_cap, g.prefix_cap / s->chunk) != hipSuccess)
    return LOWRAM_ERR_HIP;
  if (!mark(4)) return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}
}  // namespace

int lowram_build_layer(const lowram_build_shape* s, int32_t layer_in_group, const lowram_layer_build* io,
                       void* workspace, size_t ws_bytes, void* stream) {
  return run_build_layer(s, layer_in_group, io, workspace, ws_bytes, stream, nullptr);
}

int lowram_build_layer_events(const lowram_build_shape* s, int32_t layer_in_group, const lowram_layer_build* io,
                              void* workspace, size_t ws_bytes, void* stream, void* const* events) {
  return run_build_layer(s, layer_in_group, io, workspace, ws_bytes, stream, events);
}

}  // extern "C"

namespace {
int check_append(const lowram_shape* s, int32_t group_layers) {
  int st = check_shape(s);
  if (st) return st;
  if (group_layers < 1) return LOWRAM_ERR_SHAPE;
  if (!s->prefix_cap || s->prefix_len + s->chunk > s->prefix_cap) return LOWRAM_ERR_SHAPE;  // no room
  if (s->window < s->chunk) return LOWRAM_ERR_SHAPE;
  if (s->n_cand != s->prefix_len / s->chunk) return LOWRAM_ERR_SHAPE;  // no eviction
  if ((int64_t)group_layers * s->n_heads_kv * kHeadDim >= (int64_t)1 << 20) return LOWRAM_ERR_UNSUPPORTED;
  return LOWRAM_OK;
}
}  // namespace

extern "C" {

int lowram_append_coeff(const lowram_shape* shape, int32_t group_layers, const uint16_t* keys_new,
                        const uint16_t* basis, void* coeff, uint16_t* coeff_scale, void* stream) {
  int st = check_append(shape, group_layers);
  if (st) return st;
  const bool ci4 = shape->coeff_fmt == LOWRAM_FMT_INT4_G32;
  if (!keys_new || !basis || !coeff || (ci4 && !coeff_scale)) return LOWRAM_ERR_NULL;
  if (misaligned(keys_new, 16) || misaligned(basis, 16) || misaligned(coeff, 16) ||
      (coeff_scale && misaligned(coeff_scale, 4)))
    return LOWRAM_ERR_ALIGN;
  const int D = group_layers * shape->n_heads_kv * kHeadDim;
  if (launch_proj(keys_new, basis, coeff, coeff_scale, shape->batch, shape->chunk, shape->chunk, D, shape->rank,
                  ci4, static_cast<hipStream_t>(stream), shape->prefix_cap, shape->prefix_len) != hipSuccess)
    return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}

int lowram_append_layer(const lowram_shape* shape, int32_t group_layers, int32_t layer_in_group,
                        const lowram_layer_cache* cache, const lowram_layer_append* io, void* stream) {
  int st = check_append(shape, group_layers);
  if (st) return st;
  if (layer_in_group < 0 || layer_in_group >= group_layers) return LOWRAM_ERR_SHAPE;
  if (!cache || !io) return LOWRAM_ERR_NULL;
  const bool ci4 = shape->coeff_fmt == LOWRAM_FMT_INT4_G32, ri4 = shape->resid_fmt == LOWRAM_FMT_INT4_G32;
  if (!cache->coeff || !cache->basis || !cache->w1 || !cache->b1 || !cache->w2 || !cache->b2 || !io->keys_new ||
      !io->res_thresh || !io->res_count || !io->res_dropped || !io->landmark || !io->res_chunk_desc ||
      !io->win_k || !io->win_v)
    return LOWRAM_ERR_NULL;
  if (ci4 && !cache->coeff_scale) return LOWRAM_ERR_NULL;
  if (shape->n_resid > 0 && (!io->res_idx || !io->res_val || (ri4 && !io->res_scale))) return LOWRAM_ERR_NULL;
  const void* bulk[] = {cache->coeff, cache->basis, cache->w1, cache->w2, io->keys_new, io->landmark, io->res_val,
                        io->win_k, io->win_v};
  for (const void* ptr : bulk)
    if (ptr && misaligned(ptr, 16)) return LOWRAM_ERR_ALIGN;
  const void* small[] = {cache->coeff_scale, cache->b1, cache->b2, io->res_thresh, io->res_count, io->res_dropped,
                         io->res_idx, io->res_scale, io->res_chunk_desc};
  for (const void* ptr : small)
    if (ptr && misaligned(ptr, 4)) return LOWRAM_ERR_ALIGN;
  AppendArgs a{};
  a.keys_new = io->keys_new; a.coeff = cache->coeff; a.coeff_scale = cache->coeff_scale; a.blk = cache->basis;
  a.w1 = cache->w1; a.b1 = cache->b1; a.w2 = cache->w2; a.b2 = cache->b2; a.thresh = io->res_thresh;
  a.landmark = io->landmark; a.res_idx = io->res_idx; a.res_val = io->res_val; a.res_scale = io->res_scale;
  a.desc = io->res_chunk_desc; a.count = io->res_count; a.dropped = io->res_dropped;
  a.win_k = io->win_k; a.win_v = io->win_v;
  a.D = group_layers * shape->n_heads_kv * kHeadDim; a.r = shape->rank; a.hkv = shape->n_heads_kv;
  a.layer_in_group = layer_in_group; a.P = shape->prefix_len; a.W = shape->window;
  a.prefix_cap = shape->prefix_cap; a.window_cap = window_rows(shape); a.resid_cap = shape->n_resid;
  a.ci4 = ci4; a.ri4 = ri4;
  for (int i = 0; i < 64; ++i) a.inv_freq[i] = std::pow((double)shape->rope_theta, -2.0 * i / (double)kHeadDim);
  if (launch_append(a, shape->batch, static_cast<hipStream_t>(stream)) != hipSuccess) return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}

}  // extern "C"

namespace {
int check_fit(const lowram_fit_shape* s) {
  if (!s) return LOWRAM_ERR_NULL;
  if (s->batch < 1 || s->ctx_len < 1 || s->prefix_len < 1 || s->prefix_len > s->ctx_len || s->group_dim < 1 ||
      s->rank < 1 || s->power < 0)
    return LOWRAM_ERR_SHAPE;
  if (s->prefix_len % 64 || s->group_dim % 128) return LOWRAM_ERR_UNSUPPORTED;
  if (s->rank != 64 && s->rank != 128 && s->rank != 256 && s->rank != 512) return LOWRAM_ERR_UNSUPPORTED;
  if (s->rank > s->group_dim || s->rank > s->prefix_len) return LOWRAM_ERR_SHAPE;
  if (s->power > 4) return LOWRAM_ERR_UNSUPPORTED;
  if ((int64_t)s->ctx_len * s->group_dim >= (int64_t)1 << 31 || (int64_t)s->prefix_len * s->rank >= (int64_t)1 << 31)
    return LOWRAM_ERR_UNSUPPORTED;
  if (s->batch > 65535) return LOWRAM_ERR_UNSUPPORTED;  // a grid dimension of at most 65535
  // the transposes index 64-column blocks of the keys in a grid dimension of
  // at most 65535
  if (s->group_dim >= (1 << 20)) return LOWRAM_ERR_UNSUPPORTED;
  return LOWRAM_OK;
}
}  // namespace

extern "C" {

int lowram_fit_basis_workspace_bytes(const lowram_fit_shape* shape, size_t* bytes) {
  if (!bytes) return LOWRAM_ERR_NULL;
  const int st = check_fit(shape);
  if (st) return st;
  *bytes = fit_basis_ws_bytes(shape->prefix_len, shape->group_dim, shape->rank);
  return LOWRAM_OK;
}

int lowram_fit_basis(const lowram_fit_shape* shape, const uint16_t* keys, const uint16_t* omega_t, uint16_t* basis,
                     int32_t* status, void* workspace, size_t ws_bytes, void* stream) {
  int st = check_fit(shape);
  if (st) return st;
  if (!keys || !omega_t || !basis || !status || !workspace) return LOWRAM_ERR_NULL;
  if (misaligned(keys, 16) || misaligned(omega_t, 16) || misaligned(basis, 16) || misaligned(workspace, 256) ||
      misaligned(status, 4))
    return LOWRAM_ERR_ALIGN;
  if (ws_bytes < fit_basis_ws_bytes(shape->prefix_len, shape->group_dim, shape->rank)) return LOWRAM_ERR_WORKSPACE;
  if (launch_fit_basis(keys, omega_t, basis, shape->batch, shape->ctx_len, shape->prefix_len, shape->group_dim,
                       shape->rank, shape->power, workspace, status, static_cast<hipStream_t>(stream)) != hipSuccess)
    return LOWRAM_ERR_HIP;
  return LOWRAM_OK;
}

}  // extern "C"

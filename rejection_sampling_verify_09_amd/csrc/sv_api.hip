// Host side of libspecverify: argument validation, scratch management and
// kernel dispatch for the C ABI declared in include/specverify.h.
#include "sv_common.hpp"
#include "specverify.h"

#include <algorithm>
#include <cfloat>
#include <cmath>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <utility>

namespace sv {
hipError_t launch_stream(const Args& a, int dtype, int mode, bool vec, unsigned grid, hipStream_t s,
                         hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
hipError_t launch_row(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s);
hipError_t launch_seq(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s);
hipError_t launch_sample(const Args& a, int dtype, unsigned grid, hipStream_t s);
hipError_t launch_probs(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s);
hipError_t launch_read(const void* p, int64_t nbytes, uint32_t key, uint32_t* out, unsigned grid, hipStream_t s);
hipError_t launch_lm_gemm(const void* H, const void* W, float* C, int32_t M, int32_t V, int32_t d, hipStream_t s,
                          void* R, int32_t rstride, int32_t roff, int stat, float c2);
hipError_t launch_tile_chunk(const Args& a, int mode, unsigned grid, const void* R, int32_t rstride, int32_t ntg,
                             hipStream_t s);
int64_t lm_gemm_tiles(int32_t M, int32_t V);
}  // namespace sv

using namespace sv;

namespace {

constexpr int kMaxDevices = 64;
// A launch must satisfy grid * WG < 2^32.
constexpr int64_t kMaxGrid = (int64_t(1) << 32) / WG - 1;

// Scratch of the verification calls and the projection logits of
// sv_spec_verify_lmhead, one set per (device, stream): calls on different
// streams never share memory.  A call holds its set's mutex from the look-up
// to its last launch, so a growth on another host thread (same stream) waits
// for it; a growth synchronises only that stream (the only work that can
// still use the old buffer) before freeing it.  Entries live until the
// process ends (sv_release frees their memory, not the entries, so a pointer
// a concurrent call already holds stays valid).
struct StreamBufs {
  std::mutex mu;
  char* ptr = nullptr;   // verification scratch
  size_t bytes = 0;
  char* lgt = nullptr;   // float32 logits formed by the output projections, then their tile records
  size_t lgt_bytes = 0;
};

std::mutex g_mu;  // guards g_bufs (the map, not the buffers) and g_static
std::map<std::pair<int, uintptr_t>, std::unique_ptr<StreamBufs>> g_bufs;

StreamBufs* bufs_for(int dev, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto& e = g_bufs[{dev, (uintptr_t)s}];
  if (!e) e.reset(new (std::nothrow) StreamBufs());
  return e.get();
}

// Grows *p to at least `want` bytes (the caller holds the set's mutex).
int grow(char** p, size_t* have, size_t want, hipStream_t s) {
  if (*have >= want && *p) return SV_OK;
  if (*p) {
    if (hipStreamSynchronize(s) != hipSuccess) return SV_ERR_HIP;
    (void)hipFree(*p);
    *p = nullptr;
    *have = 0;
  }
  void* q = nullptr;
  if (hipMalloc(&q, want) != hipSuccess) return SV_ERR_WORKSPACE;
  *p = (char*)q;
  *have = want;
  return SV_OK;
}

// The no-allocation entry point's scratch: one array per device, placed by
// the loader with the library's code, at its own address on each device.
// The host only ever uses the address hipGetSymbolAddress returns for the
// current device (g_static), never the array's name.
static __device__ __align__(256) char scratch[SV_NOALLOC_SCRATCH_BYTES];
char* g_static[kMaxDevices];

// The device address of `scratch` on device dev (resolved once per device,
// with that device current).
int static_scratch(int dev, char** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_static[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SV_ERR_HIP;
    g_static[dev] = (char*)ptr;
  }
  *out = g_static[dev];
  return SV_OK;
}

int current_device(int* dev) {
  if (hipGetDevice(dev) != hipSuccess || *dev < 0 || *dev >= kMaxDevices) return SV_ERR_HIP;
  return SV_OK;
}

// Launch timing (sv_profile_start / sv_profile_stop): three events per call:
// the streaming kernel's start and end (recorded by its launch), and one
// recorded on the call's stream after the call's last kernel.  Slots are
// reused round-robin; a slot is folded into the totals (synchronising on its
// last event) before reuse.
constexpr int kProfSlots = 1024;
struct ProfSlot {
  hipEvent_t ev[3] = {nullptr, nullptr, nullptr};
  bool pending = false;
};
struct Profile {
  bool on = false;
  int next = 0;
  double stream_ms = 0.0, rest_ms = 0.0;
  int64_t calls = 0;
  ProfSlot slot[kProfSlots];
};
std::mutex g_prof_mu;
Profile g_prof;

// Folds a recorded slot into the totals (caller holds g_prof_mu).
int prof_fold(ProfSlot& sl) {
  if (!sl.pending) return SV_OK;
  sl.pending = false;
  float a = 0.f, b = 0.f;
  if (hipEventSynchronize(sl.ev[2]) != hipSuccess || hipEventElapsedTime(&a, sl.ev[0], sl.ev[1]) != hipSuccess ||
      hipEventElapsedTime(&b, sl.ev[1], sl.ev[2]) != hipSuccess)
    return SV_ERR_HIP;
  g_prof.stream_ms += a;
  g_prof.rest_ms += b;
  g_prof.calls += 1;
  return SV_OK;
}

// Takes the next slot for a call (nullptr when timing is off).
ProfSlot* prof_begin() {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof.on) return nullptr;
  ProfSlot& sl = g_prof.slot[g_prof.next];
  g_prof.next = (g_prof.next + 1) % kProfSlots;
  if (prof_fold(sl) != SV_OK) return nullptr;
  // timing only: no system-scope fence (cache writeback and invalidation)
  // when an event is reached, which would add to the measured launches
  for (hipEvent_t& e : sl.ev)
    if (!e && hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return &sl;
}

size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

// The projection-fed call's buffer: rows x V float32 logits, then the tile
// records of those rows (8 bytes per row and TILE_N columns, in groups of
// TILE_GROUP tiles).
size_t lm_logit_bytes(int64_t rows, int64_t V) { return al256((size_t)rows * (size_t)V * sizeof(float)); }
size_t lm_buf_bytes(int64_t rows, int64_t V) {
  const int64_t groups = (V + TILE_N * TILE_GROUP - 1) / (TILE_N * TILE_GROUP);
  return lm_logit_bytes(rows, V) + al256((size_t)groups * (size_t)rows * TILE_GROUP * sizeof(uint2));
}

// Tile records that stand in for the streaming pass (launch_plan).
struct TileIn {
  const void* R;
  int32_t rstride, ntg;
};

struct Layout {
  size_t seq_cnt, smp_cnt, cflag, chunk, ctop, cand, row, kidx, kprob, seq, seg_sum, seg_last, qxs, total;
};

// What one call needs from the scratch.
struct Need {
  int64_t rows = 0, nchunks = 0, B = 0, nseg = 0;  // nseg: sampling segments per sequence
  bool filt = false;                               // candidate and kept lists
  bool topk = false;                               // the chunks' largest thread maxima
};

// Arrival counters (cleared by each call's streaming kernel), then the data
// records of the call.  Every region's size grows with each field of Need, so
// a buffer laid out for larger bounds holds any call within them.
Layout make_layout(const Need& n) {
  Layout L;
  size_t o = 0;
  L.seq_cnt = o; o += al256(n.B * 4);
  L.smp_cnt = o; o += al256(n.B * 4);
  L.cflag = o; o += al256(4);
  L.chunk = o; o += al256(n.rows * n.nchunks * sizeof(ChunkRec));
  L.ctop = o; o += n.topk ? al256(n.rows * n.nchunks * CTOP * sizeof(uint32_t)) : 0;
  L.cand = o; o += n.filt ? al256(n.rows * n.nchunks * CAND_CAP * sizeof(uint64_t)) : 0;
  L.row = o; o += al256(n.rows * sizeof(RowRec));
  L.kidx = o; o += n.filt ? al256(n.rows * KEEP_CAP * sizeof(int32_t)) : 0;
  L.kprob = o; o += n.filt ? al256(n.rows * KEEP_CAP * sizeof(double)) : 0;
  L.seq = o; o += al256(n.B * sizeof(SeqRec));
  L.seg_sum = o; o += al256(n.B * n.nseg * sizeof(double));
  L.seg_last = o; o += al256(n.B * n.nseg * sizeof(int32_t));
  L.qxs = o; o += al256(n.rows * sizeof(float));
  L.total = o;
  return L;
}

void bind_scratch(Args& a, char* base, const Layout& L) {
  a.seq_cnt = (uint32_t*)(base + L.seq_cnt);
  a.smp_cnt = (uint32_t*)(base + L.smp_cnt);
  a.cflag = (int32_t*)(base + L.cflag);
  a.chunk = (ChunkRec*)(base + L.chunk);
  a.ctop = (uint32_t*)(base + L.ctop);
  a.cand = (uint64_t*)(base + L.cand);
  a.row = (RowRec*)(base + L.row);
  a.kidx = (int32_t*)(base + L.kidx);
  a.kprob = (double*)(base + L.kprob);
  a.seq = (SeqRec*)(base + L.seq);
  a.seg_sum = (double*)(base + L.seg_sum);
  a.seg_last = (int32_t*)(base + L.seg_last);
  a.qxs = (float*)(base + L.qxs);
}

int check_params(float T, int32_t top_k, float top_p) {
  if (!(T >= 0.0f) || !std::isfinite(T) || (T > 0.0f && T < FLT_MIN)) return SV_ERR_PARAM;
  if (top_k < 0) return SV_ERR_PARAM;
  if (!(top_p > 0.0f && top_p <= 1.0f)) return SV_ERR_PARAM;
  return SV_OK;
}

int pick_mode(float T, int32_t top_k, float top_p, int32_t V) {
  if (T == 0.0f) return M_GREEDY;
  const bool k = top_k > 0 && top_k < V;
  const bool p = top_p < 1.0f;
  return k && p ? M_TOPKP : k ? M_TOPK : p ? M_TOPP : M_PLAIN;
}

void temp_scalars(float T, float* c2, float* win, double* invT) {
  if (T > 0.0f) {
    *invT = 1.0 / (double)T;
    *c2 = (float)(1.4426950408889634074 / (double)T);
    *win = TOPP_WINDOW_Z * T;
  } else {
    *invT = 0.0;
    *c2 = 0.0f;
    *win = 0.0f;
  }
}

// Td: the draft rows' temperature (the target's unless the drafts were
// sampled at another one).
void set_scalars(Args& a, float T, int32_t top_k, float top_p, float Td) {
  a.top_k = top_k;
  a.top_p = (double)top_p;
  temp_scalars(T, &a.c2, &a.win, &a.invT);
  temp_scalars(T > 0.0f ? Td : T, &a.c2d, &a.wind, &a.invTd);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A ragged batch: per-sequence draft counts from device offsets cu[B + 1]
// (nd drafts in total, at most kmax per sequence).
struct Ragged {
  const int32_t* cu;
  int32_t nd, kmax;
};

// One verification call's inputs.  need_n: out_n is required (the sampler
// passes none).  out_px: probability of each sequence's last drawn token under
// the row it was drawn from (the sampler, K == 0).  rg: null for a
// rectangular [B, K] batch.  qp / qprob: the draft distributions given as
// probabilities [B, K, V] (rectangular only; drf is then not used).
struct VerifyIn {
  const void* tgt = nullptr;
  const void* drf = nullptr;
  const int32_t* X = nullptr;
  const float* U = nullptr;
  float T = 1.0f, Td = 1.0f;
  int32_t top_k = 0;
  float top_p = 1.0f;
  int32_t* out_tok = nullptr;
  int32_t* out_n = nullptr;
  bool need_n = true;
  double *out_p = nullptr, *out_q = nullptr, *out_z = nullptr, *out_px = nullptr;
  int32_t B = 0, K = 0, V = 0, dtype = 0;
  const Ragged* rg = nullptr;
  const float* qprob = nullptr;
  bool qp = false;
};

// A validated call: its kernel arguments (all but the scratch pointers), its
// launch grids and its scratch needs.
struct Plan {
  Args a;
  int mode = 0, dtype = 0;
  bool vec = false;
  unsigned g_stream = 0, g_seq = 0, g_sample = 0;
  Need need;
  bool empty = false;  // B == 0: nothing to launch
};

int plan_verify(const VerifyIn& in, Plan* p) {
  const int32_t B = in.B, K = in.K, V = in.V;
  const Ragged* rg = in.rg;
  if (B < 0 || K < 0 || K > SV_MAX_K || V < 1 || V > MAX_V) return SV_ERR_SHAPE;
  if (rg && (rg->nd < 0 || rg->kmax < 0 || rg->kmax > SV_MAX_K || (int64_t)rg->nd > (int64_t)B * rg->kmax))
    return SV_ERR_SHAPE;
  if (in.dtype != SV_F32 && in.dtype != SV_BF16) return SV_ERR_DTYPE;
  int st = check_params(in.T, in.top_k, in.top_p);
  if (st != SV_OK) return st;
  // at T > 0 the draft temperature must be a valid temperature above 0
  if (in.T > 0.0f && (check_params(in.Td, in.top_k, in.top_p) != SV_OK || !(in.Td > 0.0f))) return SV_ERR_PARAM;
  if (B == 0) {
    p->empty = true;
    return SV_OK;
  }
  const int mode = pick_mode(in.T, in.top_k, in.top_p, V);
  const int64_t nd = rg ? rg->nd : (int64_t)B * K;  // draft rows
  const int32_t kmax = rg ? rg->kmax : K;
  if (!in.tgt || !in.U || !in.out_tok || (in.need_n && !in.out_n) || (rg && !rg->cu)) return SV_ERR_NULL;
  if (nd > 0 && !in.X) return SV_ERR_NULL;
  if (nd > 0 && mode != M_GREEDY && !(in.qp ? (const void*)in.qprob : in.drf)) return SV_ERR_NULL;
  // q given as probabilities: no draft rows to stream (greedy never uses q)
  const bool use_qp = in.qp && mode != M_GREEDY && nd > 0;
  const int esz = in.dtype == SV_BF16 ? 2 : 4;
  const int64_t nt = nd + B;  // target rows
  const int64_t rows = (mode == M_GREEDY || use_qp) ? nt : nt + nd;
  const int64_t nchunks = ((int64_t)V + CE - 1) / CE;
  const int64_t nsc = ((int64_t)V + SCE - 1) / SCE;
  if ((rows + NXCD) * nchunks > kMaxGrid || (int64_t)B * nsc > kMaxGrid) return SV_ERR_SHAPE;
  Need& need = p->need;
  need.rows = rows;
  need.nchunks = nchunks;
  need.B = B;
  need.nseg = nsc * SEG_PER_SCE;
  need.filt = mode == M_TOPK || mode == M_TOPP || mode == M_TOPKP;
  need.topk = mode == M_TOPK || mode == M_TOPKP;

  Args& a = p->a;
  a = Args{};
  a.tgt = in.tgt;
  a.drf = (mode == M_GREEDY || use_qp) ? nullptr : in.drf;
  a.qprob = use_qp ? in.qprob : nullptr;
  a.X = in.X;
  a.U = in.U;
  a.out_tok = in.out_tok;
  a.out_n = in.out_n;
  a.out_p = in.out_p;
  a.out_q = in.out_q;
  a.out_z = in.out_z;
  a.out_px = in.out_px;
  a.out_probs = nullptr;
  a.B = B;
  a.K = rg ? 0 : K;
  a.V = V;
  a.NT = (int32_t)nt;
  a.ND = (int32_t)nd;
  a.Kmax = kmax;
  a.cu = rg ? rg->cu : nullptr;
  a.nchunks = (int32_t)nchunks;
  a.nsc = (int32_t)nsc;
  // sampling chunks per workgroup: up to SPW (fewer, longer workgroups
  // measured faster), while at least one workgroup per compute unit remains
  a.spw = (int32_t)std::max<int64_t>(1, std::min<int64_t>(SPW, (int64_t)B * nsc / 256));
  a.nsw = (int32_t)((nsc + a.spw - 1) / a.spw);
  a.do_seq = 1;
  set_scalars(a, in.T, in.top_k, in.top_p, in.Td);
  const bool vec = aligned16(in.tgt) && (a.drf == nullptr || aligned16(a.drf)) && ((int64_t)V * esz) % 16 == 0;
  a.ulen = vec ? 16 / esz : 1;
  a.dch = make_udiv((uint32_t)a.nchunks);
  a.rps = rg ? 1 : (mode == M_GREEDY || use_qp) ? a.K + 1 : 2 * a.K + 1;
  a.drps = make_udiv((uint32_t)a.rps);
  p->mode = mode;
  p->dtype = in.dtype;
  p->vec = vec;
  a.nitems = (int32_t)(rows * nchunks);
  p->g_stream = (unsigned)(((rows + NXCD - 1) / NXCD) * NXCD * nchunks);
  p->g_seq = (unsigned)B;
  p->g_sample = mode == M_PLAIN ? (unsigned)((int64_t)B * a.nsw) : 0u;
  return SV_OK;
}

// Binds the call to scratch at `base` (at least make_layout(need).total
// bytes) and enqueues its kernels: the chunk-parallel streaming pass, then one
// workgroup per sequence merges the sequence's rows and finishes it (accept
// tests, first rejection, draw), then for unfiltered rows the full-row draw.  When timing, the
// streaming launch records its own start and end in the slot's events.
int launch_plan(Plan& p, char* base, hipStream_t s, ProfSlot* prof, const TileIn* tiles = nullptr) {
  bind_scratch(p.a, base, make_layout(p.need));
  if (tiles) {
    // the chunk records from the projections' tile statistics (the rows
    // are already in HBM; only the candidate tiles are read back)
    if (launch_tile_chunk(p.a, p.mode, p.g_stream, tiles->R, tiles->rstride, tiles->ntg, s) != hipSuccess)
      return SV_ERR_HIP;
  } else if (launch_stream(p.a, p.dtype, p.mode, p.vec, p.g_stream, s, prof ? prof->ev[0] : nullptr,
                           prof ? prof->ev[1] : nullptr) != hipSuccess) {
    return SV_ERR_HIP;
  }
  if (launch_seq(p.a, p.dtype, p.mode, p.g_seq, s) != hipSuccess) return SV_ERR_HIP;
  if (p.g_sample > 0 && launch_sample(p.a, p.dtype, p.g_sample, s) != hipSuccess) return SV_ERR_HIP;
  if (prof) {
    if (hipEventRecord(prof->ev[2], s) != hipSuccess) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    prof->pending = true;
  }
  return SV_OK;
}

// A planned call on the stream's own scratch; the caller holds b->mu.
int run_plan_locked(Plan& p, StreamBufs* b, hipStream_t s, bool timed, const TileIn* tiles = nullptr) {
  int st = grow(&b->ptr, &b->bytes, make_layout(p.need).total, s);
  if (st != SV_OK) return st;
  ProfSlot* prof = timed ? prof_begin() : nullptr;
  return launch_plan(p, b->ptr, s, prof, tiles);
}

int verify_impl(const VerifyIn& in, void* stream, bool timed = true) {
  Plan p;
  int st = plan_verify(in, &p);
  if (st != SV_OK || p.empty) return st;
  int dev = 0;
  if ((st = current_device(&dev)) != SV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  StreamBufs* b = bufs_for(dev, s);
  if (!b) return SV_ERR_WORKSPACE;
  std::lock_guard<std::mutex> lk(b->mu);
  return run_plan_locked(p, b, s, timed);
}

// Top-p candidate window (units of z = logit / T below the chunk max) on
// rows whose chunk records come from the projections' tile records, where a
// wider window costs only the tiles it reaches.  The flatter tops of
// projection-fed rows put a few nuclei just past the streaming path's 5
// units, and each such row takes the block-level merge; 6 measured best on
// those rows (wider windows overflow the candidate lists instead).
constexpr float TOPP_WINDOW_Z_TILES = 6.0f;

// Largest hidden width accepted (the kernel needs only d % 64 == 0).
constexpr int32_t kMaxHidden = 1 << 16;

int check_lm_shape(const void* H, const void* W, int64_t M, int32_t V, int32_t d) {
  if (M < 0 || V < 1 || V > MAX_V || d < 64 || d > kMaxHidden || d % 64 != 0) return SV_ERR_SHAPE;
  if (M > 0 && (!H || !W)) return SV_ERR_NULL;
  if (M > 0 && (!aligned16(H) || !aligned16(W))) return SV_ERR_SHAPE;
  if (M > INT32_MAX || sv::lm_gemm_tiles((int32_t)std::min<int64_t>(M, INT32_MAX), V) > kMaxGrid) return SV_ERR_SHAPE;
  return SV_OK;
}

}  // namespace

extern "C" {

int sv_lm_logits(const void* hidden, const void* weight, float* out_logits, int32_t M, int32_t V, int32_t d,
                 void* stream) {
  int st = check_lm_shape(hidden, weight, M, V, d);
  if (st != SV_OK) return st;
  if (M == 0) return SV_OK;
  if (!out_logits) return SV_ERR_NULL;
  return launch_lm_gemm(hidden, weight, out_logits, M, V, d, (hipStream_t)stream, nullptr, 0, 0, TS_NONE, 0.0f) ==
                 hipSuccess
             ? SV_OK
             : SV_ERR_HIP;
}

int sv_spec_verify_lmhead(const void* hidden_target, const void* weight_target, const void* hidden_draft,
                          const void* weight_draft, const int32_t* draft_tokens, const float* uniforms,
                          float temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                          int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z, int32_t B,
                          int32_t K, int32_t V, int32_t d_target, int32_t d_draft, void* stream) {
  if (B < 0 || K < 0 || K > SV_MAX_K) return SV_ERR_SHAPE;
  int st = check_params(temperature, top_k, top_p);
  if (st != SV_OK) return st;
  const bool greedy = temperature == 0.0f;
  const int64_t mt = (int64_t)B * (K + 1), md = greedy ? 0 : (int64_t)B * K;
  st = check_lm_shape(hidden_target, weight_target, mt, V, d_target);
  if (st != SV_OK) return st;
  if (md > 0 && (st = check_lm_shape(hidden_draft, weight_draft, md, V, d_draft)) != SV_OK) return st;
  if (B == 0) return SV_OK;
  if (!uniforms || !out_tokens || !out_num_accepted || (K > 0 && !draft_tokens)) return SV_ERR_NULL;
  int dev = 0;
  if ((st = current_device(&dev)) != SV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  StreamBufs* b = bufs_for(dev, s);
  if (!b) return SV_ERR_WORKSPACE;
  std::lock_guard<std::mutex> lk(b->mu);
  st = grow(&b->lgt, &b->lgt_bytes, lm_buf_bytes(mt + md, V), s);
  if (st != SV_OK) return st;
  float* lt = (float*)b->lgt;
  float* ld = md > 0 ? lt + (size_t)mt * V : nullptr;
  // Rows of 16 bytes' multiple (V % 4 == 0) take the fused path: the
  // projections' epilogues write tile records beside the logits, and the
  // chunk records are formed from them instead of a streaming pass over the
  // logits.  Other rows are streamed (the element-load path).
  const bool fused = V % 4 == 0;
  TileIn tiles{b->lgt + lm_logit_bytes(mt + md, V), (int32_t)(mt + md), (V + TILE_N - 1) / TILE_N};
  const int stat = !fused ? TS_NONE : greedy ? TS_ARG : TS_SUM;
  void* R = fused ? const_cast<void*>(tiles.R) : nullptr;
  VerifyIn in;
  in.tgt = lt;
  in.drf = ld;
  in.X = draft_tokens;
  in.U = uniforms;
  in.T = in.Td = temperature;
  in.top_k = top_k;
  in.top_p = top_p;
  in.out_tok = out_tokens;
  in.out_n = out_num_accepted;
  in.out_p = out_p;
  in.out_q = out_q;
  in.out_z = out_z;
  in.B = B;
  in.K = K;
  in.V = V;
  in.dtype = SV_F32;
  Plan p;
  if ((st = plan_verify(in, &p)) != SV_OK) return st;
  if (fused && temperature > 0.0f) p.a.win = p.a.wind = TOPP_WINDOW_Z_TILES * temperature;
  // when timing, the slot's first two events bracket the two projections and
  // the third follows the verification
  ProfSlot* prof = prof_begin();
  if (prof && hipEventRecord(prof->ev[0], s) != hipSuccess) return SV_ERR_HIP;
  if (launch_lm_gemm(hidden_target, weight_target, lt, (int32_t)mt, V, d_target, s, R, tiles.rstride, 0, stat,
                     p.a.c2) != hipSuccess)
    return SV_ERR_HIP;
  if (md > 0 && launch_lm_gemm(hidden_draft, weight_draft, ld, (int32_t)md, V, d_draft, s, R, tiles.rstride,
                               (int32_t)mt, stat, p.a.c2d) != hipSuccess)
    return SV_ERR_HIP;
  if (prof && hipEventRecord(prof->ev[1], s) != hipSuccess) return SV_ERR_HIP;
  st = run_plan_locked(p, b, s, false, fused ? &tiles : nullptr);
  if (st != SV_OK) return st;
  if (prof) {
    if (hipEventRecord(prof->ev[2], s) != hipSuccess) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lk2(g_prof_mu);
    prof->pending = true;
  }
  return SV_OK;
}

static VerifyIn verify_in(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                          const float* uniforms, float temperature, float draft_temperature, int32_t top_k,
                          float top_p, int32_t* out_tokens, int32_t* out_num_accepted, double* out_p, double* out_q,
                          double* out_z, int32_t B, int32_t K, int32_t V, int32_t dtype) {
  VerifyIn in;
  in.tgt = target_logits;
  in.drf = draft_logits;
  in.X = draft_tokens;
  in.U = uniforms;
  in.T = temperature;
  in.Td = draft_temperature;
  in.top_k = top_k;
  in.top_p = top_p;
  in.out_tok = out_tokens;
  in.out_n = out_num_accepted;
  in.out_p = out_p;
  in.out_q = out_q;
  in.out_z = out_z;
  in.B = B;
  in.K = K;
  in.V = V;
  in.dtype = dtype;
  return in;
}

int sv_spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                   const float* uniforms, float temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                   int32_t* out_num_accepted, int32_t B, int32_t K, int32_t V, int32_t dtype, void* stream) {
  return verify_impl(verify_in(target_logits, draft_logits, draft_tokens, uniforms, temperature, temperature, top_k,
                               top_p, out_tokens, out_num_accepted, nullptr, nullptr, nullptr, B, K, V, dtype),
                     stream);
}

int sv_spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                           const float* uniforms, float temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                           int32_t* out_num_accepted, int32_t B, int32_t K, int32_t V, int32_t dtype, void* stream) {
  Plan p;
  int st = plan_verify(verify_in(target_logits, draft_logits, draft_tokens, uniforms, temperature, temperature,
                                 top_k, top_p, out_tokens, out_num_accepted, nullptr, nullptr, nullptr, B, K, V,
                                 dtype),
                       &p);
  if (st != SV_OK || p.empty) return st;
  if (make_layout(p.need).total > (size_t)SV_NOALLOC_SCRATCH_BYTES) return SV_ERR_WORKSPACE;
  int dev = 0;
  char* base = nullptr;
  if ((st = current_device(&dev)) != SV_OK || (st = static_scratch(dev, &base)) != SV_OK) return st;
  return launch_plan(p, base, (hipStream_t)stream, nullptr);
}

int sv_spec_verify_debug(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                         const float* uniforms, float temperature, int32_t top_k, float top_p,
                         int32_t* out_tokens, int32_t* out_num_accepted, double* out_p, double* out_q,
                         double* out_z, int32_t B, int32_t K, int32_t V, int32_t dtype, void* stream) {
  return verify_impl(verify_in(target_logits, draft_logits, draft_tokens, uniforms, temperature, temperature, top_k,
                               top_p, out_tokens, out_num_accepted, out_p, out_q, out_z, B, K, V, dtype),
                     stream);
}

int sv_spec_verify_dt(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                      const float* uniforms, float temperature, float draft_temperature, int32_t top_k, float top_p,
                      int32_t* out_tokens, int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z,
                      int32_t B, int32_t K, int32_t V, int32_t dtype, void* stream) {
  return verify_impl(verify_in(target_logits, draft_logits, draft_tokens, uniforms, temperature, draft_temperature,
                               top_k, top_p, out_tokens, out_num_accepted, out_p, out_q, out_z, B, K, V, dtype),
                     stream);
}

int sv_spec_verify_ragged(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                          const float* uniforms, const int32_t* cu_num_draft, float temperature,
                          float draft_temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                          int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z, int32_t B,
                          int32_t total_draft, int32_t max_k, int32_t V, int32_t dtype, void* stream) {
  const Ragged rg{cu_num_draft, total_draft, max_k};
  VerifyIn in = verify_in(target_logits, draft_logits, draft_tokens, uniforms, temperature, draft_temperature, top_k,
                          top_p, out_tokens, out_num_accepted, out_p, out_q, out_z, B, 0, V, dtype);
  in.rg = &rg;
  return verify_impl(in, stream);
}

int sv_spec_verify_probs(const void* target_logits, const float* draft_probs, const int32_t* draft_tokens,
                         const float* uniforms, float temperature, int32_t top_k, float top_p, int32_t* out_tokens,
                         int32_t* out_num_accepted, double* out_p, double* out_q, double* out_z, int32_t B, int32_t K,
                         int32_t V, int32_t dtype, void* stream) {
  VerifyIn in = verify_in(target_logits, nullptr, draft_tokens, uniforms, temperature, temperature, top_k, top_p,
                          out_tokens, out_num_accepted, out_p, out_q, out_z, B, K, V, dtype);
  in.qprob = draft_probs;
  in.qp = true;
  return verify_impl(in, stream);
}

// The draw of a verification with no drafts: each row is a sequence of one
// position whose only token is drawn from its own filtered distribution with
// its own uniform.
int sv_sample(const void* logits, const float* uniforms, float temperature, int32_t top_k, float top_p,
              int32_t* out_tokens, double* out_prob, int32_t rows, int32_t V, int32_t dtype, void* stream) {
  VerifyIn in = verify_in(logits, nullptr, nullptr, uniforms, temperature, temperature, top_k, top_p, out_tokens,
                          nullptr, nullptr, nullptr, nullptr, rows, 0, V, dtype);
  in.need_n = false;
  in.out_px = out_prob;
  return verify_impl(in, stream);
}

int sv_filtered_probs(const void* logits, int32_t rows, int32_t V, int32_t dtype, float temperature, int32_t top_k,
                      float top_p, float* out_probs, void* stream) {
  if (rows < 0 || V < 1 || V > MAX_V) return SV_ERR_SHAPE;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  int st = check_params(temperature, top_k, top_p);
  if (st != SV_OK) return st;
  if (temperature == 0.0f) return SV_ERR_PARAM;
  if (rows == 0) return SV_OK;
  if (!logits || !out_probs) return SV_ERR_NULL;
  const int mode = pick_mode(temperature, top_k, top_p, V);
  const int esz = dtype == SV_BF16 ? 2 : 4;
  const int64_t nchunks = ((int64_t)V + CE - 1) / CE;
  const int64_t nsc = ((int64_t)V + SCE - 1) / SCE;
  if (((int64_t)rows + NXCD) * nchunks > kMaxGrid || (int64_t)rows * nsc > kMaxGrid) return SV_ERR_SHAPE;
  Need need;
  need.rows = rows;
  need.nchunks = nchunks;
  need.B = rows;
  need.filt = mode != M_PLAIN;
  need.topk = mode == M_TOPK || mode == M_TOPKP;
  Args a = {};
  a.tgt = logits;
  a.out_probs = out_probs;
  a.B = rows;
  a.K = 0;
  a.V = V;
  a.NT = rows;
  a.nchunks = (int32_t)nchunks;
  a.nsc = (int32_t)nsc;
  a.do_seq = 0;
  set_scalars(a, temperature, top_k, top_p, temperature);
  const bool vec = aligned16(logits) && ((int64_t)V * esz) % 16 == 0;
  a.ulen = vec ? 16 / esz : 1;
  a.dch = make_udiv((uint32_t)a.nchunks);
  a.rps = 1;
  a.drps = make_udiv(1u);
  a.nitems = (int32_t)((int64_t)rows * nchunks);
  int dev = 0;
  if ((st = current_device(&dev)) != SV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  StreamBufs* b = bufs_for(dev, s);
  if (!b) return SV_ERR_WORKSPACE;
  std::lock_guard<std::mutex> lk(b->mu);
  if ((st = grow(&b->ptr, &b->bytes, make_layout(need).total, s)) != SV_OK) return st;
  bind_scratch(a, b->ptr, make_layout(need));
  if (launch_stream(a, dtype, mode, vec, (unsigned)((((int64_t)rows + NXCD - 1) / NXCD) * NXCD * nchunks), s) !=
      hipSuccess)
    return SV_ERR_HIP;
  if (launch_row(a, dtype, mode, (unsigned)rows, s) != hipSuccess) return SV_ERR_HIP;
  if (launch_probs(a, dtype, mode, (unsigned)((int64_t)rows * nsc), s) != hipSuccess) return SV_ERR_HIP;
  return SV_OK;
}

int sv_init(int device, void* stream, int32_t max_B, int32_t max_K, int32_t max_V, int32_t flags) {
  if (device < 0 || device >= kMaxDevices) return SV_ERR_PARAM;
  if (max_B < 0 || max_K < 0 || max_K > SV_MAX_K || max_V < 1 || max_V > MAX_V) return SV_ERR_SHAPE;
  if (flags & ~SV_INIT_LMHEAD) return SV_ERR_PARAM;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SV_ERR_HIP;
  if (hipSetDevice(device) != hipSuccess) return SV_ERR_HIP;
  int st = SV_OK;
  {
    // the largest call within the bounds, in every mode: its rows also bound
    // the sampler's and sv_filtered_probs' rows (each of them a sequence)
    const int64_t rows = (int64_t)max_B * (2 * (int64_t)max_K + 1);
    Need need;
    need.rows = rows;
    need.nchunks = ((int64_t)max_V + CE - 1) / CE;
    need.B = rows;
    need.nseg = (((int64_t)max_V + SCE - 1) / SCE) * SEG_PER_SCE;
    need.filt = true;
    need.topk = true;
    hipStream_t s = (hipStream_t)stream;
    StreamBufs* b = bufs_for(device, s);
    if (!b) {
      st = SV_ERR_WORKSPACE;
    } else {
      std::lock_guard<std::mutex> lk(b->mu);
      st = grow(&b->ptr, &b->bytes, std::max<size_t>(make_layout(need).total, 256), s);
      if (st == SV_OK && (flags & SV_INIT_LMHEAD))
        st = grow(&b->lgt, &b->lgt_bytes, lm_buf_bytes(rows, max_V), s);
    }
    // set-up of the no-allocation entry point on this device
    char* base = nullptr;
    if (st == SV_OK) st = static_scratch(device, &base);
  }
  if (hipSetDevice(cur) != hipSuccess && st == SV_OK) st = SV_ERR_HIP;
  return st;
}

int sv_read_floor(const void* data, int64_t nbytes, uint32_t key, uint32_t* out, void* stream) {
  if (nbytes < 0 || nbytes % 16 != 0 || (nbytes + READ_BLOCK - 1) / READ_BLOCK > kMaxGrid) return SV_ERR_SHAPE;
  if (nbytes == 0) return SV_OK;
  if (!data || !out) return SV_ERR_NULL;
  const unsigned grid = (unsigned)((nbytes + READ_BLOCK - 1) / READ_BLOCK);
  return launch_read(data, nbytes, key, out, grid, (hipStream_t)stream) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int sv_profile_start(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (ProfSlot& sl : g_prof.slot) sl.pending = false;
  g_prof.on = true;
  g_prof.next = 0;
  g_prof.stream_ms = g_prof.rest_ms = 0.0;
  g_prof.calls = 0;
  return SV_OK;
}

int sv_profile_stop(double* stream_kernel_ms, double* other_kernels_ms, int64_t* calls) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.on = false;
  int rc = SV_OK;
  for (int i = 0; i < kProfSlots; ++i) {
    ProfSlot& sl = g_prof.slot[(g_prof.next + i) % kProfSlots];
    if (prof_fold(sl) != SV_OK) rc = SV_ERR_HIP;
  }
  if (stream_kernel_ms) *stream_kernel_ms = g_prof.stream_ms;
  if (other_kernels_ms) *other_kernels_ms = g_prof.rest_ms;
  if (calls) *calls = g_prof.calls;
  return rc;
}

// Frees the memory of every (device, stream) set, after synchronising each
// device that holds one.  The sets themselves stay (empty), so a call that
// is about to use one allocates afresh.
int sv_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int rc = SV_OK;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return SV_ERR_HIP;
  bool synced[kMaxDevices] = {};
  for (auto& e : g_bufs) {
    StreamBufs* b = e.second.get();
    if (!b) continue;
    std::lock_guard<std::mutex> lb(b->mu);
    if (!b->ptr && !b->lgt) continue;
    const int d = e.first.first;
    if (hipSetDevice(d) != hipSuccess) {
      rc = SV_ERR_HIP;
      continue;
    }
    if (!synced[d]) {
      if (hipDeviceSynchronize() != hipSuccess) rc = SV_ERR_HIP;
      synced[d] = true;
    }
    if (b->ptr && hipFree(b->ptr) != hipSuccess) rc = SV_ERR_HIP;
    if (b->lgt && hipFree(b->lgt) != hipSuccess) rc = SV_ERR_HIP;
    b->ptr = b->lgt = nullptr;
    b->bytes = b->lgt_bytes = 0;
  }
  (void)hipSetDevice(cur);
  return rc;
}

int sv_stream_release(void* stream) {
  int dev = 0;
  int st = current_device(&dev);
  if (st != SV_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  StreamBufs* b = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    auto it = g_bufs.find({dev, (uintptr_t)s});
    if (it == g_bufs.end() || !it->second) return SV_OK;
    b = it->second.get();
  }
  std::lock_guard<std::mutex> lb(b->mu);
  if (!b->ptr && !b->lgt) return SV_OK;
  if (hipStreamSynchronize(s) != hipSuccess) return SV_ERR_HIP;
  if (b->ptr && hipFree(b->ptr) != hipSuccess) st = SV_ERR_HIP;
  if (b->lgt && hipFree(b->lgt) != hipSuccess) st = SV_ERR_HIP;
  b->ptr = b->lgt = nullptr;
  b->bytes = b->lgt_bytes = 0;
  return st;
}

int64_t sv_scratch_bytes(int device) {
  if (device < 0 || device >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lk(g_mu);
  int64_t total = 0;
  for (auto& e : g_bufs) {
    if (e.first.first != device || !e.second) continue;
    std::lock_guard<std::mutex> lb(e.second->mu);
    total += (int64_t)(e.second->bytes + e.second->lgt_bytes);
  }
  return total;
}

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_NULL: return "SV_ERR_NULL: a required pointer is NULL";
    case SV_ERR_SHAPE: return "SV_ERR_SHAPE: B, K or V out of range";
    case SV_ERR_DTYPE: return "SV_ERR_DTYPE: unknown logit dtype";
    case SV_ERR_PARAM: return "SV_ERR_PARAM: temperature, top_k or top_p out of range";
    case SV_ERR_HIP: return "SV_ERR_HIP: a HIP runtime call failed";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE: scratch allocation failed";
    default: return "unknown status";
  }
}

int sv_version(void) { return 200; }

}  // extern "C"

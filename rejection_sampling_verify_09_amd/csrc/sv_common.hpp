// Shared definitions of the gfx950 verification kernels: tile sizes, scratch
// records, kernel arguments and small wave/block primitives (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

namespace sv {

constexpr int WG = 256;          // threads per workgroup (4 wave64)
constexpr int NWAVE = WG / 64;
constexpr int CE = 8192;         // logits per streaming chunk
constexpr int EPT = CE / WG;     // logits held in registers per thread (32)
constexpr int CAND_CAP = 256;    // candidate slots per chunk
constexpr int KEEP_CAP = 256;    // kept-list capacity per row (one entry per thread)
constexpr int SCE = 2048;        // logits per sampling chunk (8 per thread)
constexpr int SEG = 512;         // logits per sampling segment (one wave)
constexpr int SEG_PER_SCE = SCE / SEG;
constexpr int SPW = 4;           // most sampling chunks per workgroup of the unfiltered draw
constexpr int CTOP = 8;          // top-k: largest thread maxima a chunk records for the row merge
constexpr int CTOP_CHUNKS = 64;  // ... used by the row merge for rows of at most this many chunks
constexpr int MAX_K = 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // four 32-bit words (16-byte loads and stores)
constexpr int READ_BLOCK = 16384;  // bytes per workgroup of the plain-read kernel (as a bf16 chunk)
// register budget of the streaming kernels: resident workgroups per CU
template <int DT, bool VEC>
constexpr int stream_wg_per_cu() { return VEC ? 8 : 5; }
constexpr int MAX_CHUNKS = WG;           // chunks per row (one chunk record per thread in a row merge)
constexpr int64_t MAX_V = (int64_t)MAX_CHUNKS * CE;  // 2,097,152
constexpr int MAX_RPS = 2 * MAX_K + 1;
// top-p candidates: every logit within this many units of z = logit / T below
// the row maximum (the cut is verified against the mass at the row merge)
constexpr float TOPP_WINDOW_Z = 5.0f;

enum Mode : int { M_PLAIN = 0, M_TOPK = 1, M_TOPP = 2, M_TOPKP = 3, M_GREEDY = 4 };
enum DType : int { D_F32 = 0, D_BF16 = 1 };

// Tile statistics of logits formed by the output projections: for each row
// and tile of TILE_N consecutive columns (one wave's columns of a projection
// tile), 8 bytes: the tile max (float bits) and either the sum over the tile
// of exp2(x * c2 - ceil(max * c2)) (TS_SUM, float bits) or the lowest column
// holding the max (TS_ARG).  Stored in groups of TILE_GROUP tiles (the 256
// columns of one projection workgroup): tile g of row r at
// [(g / TILE_GROUP) * rows + r] * TILE_GROUP + g % TILE_GROUP.
constexpr int TILE_N = 64;
constexpr int TILE_GROUP = 4;
constexpr int TILES_PER_CHUNK = CE / TILE_N;  // 128
enum TileStat : int { TS_NONE = 0, TS_SUM = 1, TS_ARG = 2 };

// row flags
constexpr int RF_BAD = 1;       // no distribution (all -inf or non-finite normaliser)
constexpr int RF_BIG = 2;       // kept set larger than KEEP_CAP: no kept list stored
constexpr int RF_FALLBACK = 4;  // threshold found by the full-row search

// per (row, chunk) summary, 32 bytes
struct ChunkRec {
  double s;        // sum over the chunk of exp2(x * c2), relative to 2^ceil(m * c2) (see chunk_weight)
  float m;         // chunk max logit
  uint32_t bound;  // key of the candidate threshold used by this chunk
  int32_t ncand;   // candidates found (> CAND_CAP means some were dropped)
  int32_t arg;     // lowest index of the chunk max (greedy)
  int32_t pad0, pad1;
};

// per row, 48 bytes
struct RowRec {
  double S;        // full-row normaliser sum exp((x - m) / T)
  double S_kept;   // normaliser over the kept set (filtered rows)
  double px;       // probability of the drafted token of this row
  float m;         // row max logit
  uint32_t tau;    // key threshold: token kept iff key(logit) >= tau (0 = all)
  int32_t nkept;   // kept-list length (filtered rows, valid unless RF_BIG)
  int32_t flags;
  int32_t arg;     // greedy arg-max
  int32_t pad;
};

// per sequence, 56 bytes: the outcome of the accept tests and, for the
// unfiltered draw that follows, where its rows lie and their normalisers
struct SeqRec {
  double Z;
  int32_t n;       // accepted drafts, -1 for a sentinel sequence
  int32_t flags;
  int32_t rp, rq;  // rows of p and q (q: with given probabilities, the index of its probability row)
  int32_t tu;      // index of the sequence's sampling uniform
  int32_t k;       // the sequence's number of drafts
  float mp, mq;    // row maxima of p and q
  double sp, sq;   // full-row normalisers of p and q
};

// Unsigned division by a launch constant d >= 1 as a multiply and a shift:
// with l = ceil(log2 d) and m = ceil(2^(31+l) / d) < 2^32, n / d equals
// (n * m) >> (31 + l) for every n < 2^31 (m * d - 2^(31+l) < d <= 2^l keeps
// the error below the distance to the next multiple).  Uniform operands make
// it scalar work.
struct UDiv {
  uint32_t m;
  int32_t s;
};
__host__ __device__ inline UDiv make_udiv(uint32_t d) {
  int l = 0;
  while ((1ull << l) < d) ++l;
  const unsigned long long p = 1ull << (31 + l);
  return UDiv{(uint32_t)((p + d - 1) / d), 31 + l};
}
__device__ __forceinline__ int udiv(int n, UDiv d) { return (int)(((uint64_t)(uint32_t)n * d.m) >> d.s); }

struct Args {
  const void* tgt;
  const void* drf;
  const int32_t* X;
  const float* U;
  int32_t* out_tok;
  int32_t* out_n;
  double* out_p;
  double* out_q;
  double* out_z;
  double* out_px;  // per sequence: probability of the last drawn token under the row it was drawn from
  float* out_probs;
  int32_t B, K, V;
  int32_t rps;         // rows per sequence (rectangular; 1 for ragged batches, with K = 0)
  int32_t nchunks, nsc, top_k, do_seq;
  int32_t nsw, spw;    // sampling workgroups per sequence, and sampling chunks each (at most SPW)
  // Rows are numbered in the order they are streamed, and every per-row
  // record is kept under that number.  Rectangular batches: sequence by
  // sequence, row b * rps + j is the sequence's target row j (j <= K) or
  // draft row j - K - 1.  Ragged batches (cu[B + 1] offsets, K_b = cu[b + 1]
  // - cu[b]): every target row first (sequence b's from row cu[b] + b), then
  // every draft row (its from row NT + cu[b]), which is also the order of the
  // packed inputs.
  int32_t NT;          // target rows
  int32_t ND;          // draft rows
  int32_t Kmax;        // output stride of out_tok is Kmax + 1
  const int32_t* cu;   // ragged offsets (device), or null for a rectangular batch
  const float* qprob;  // draft distributions given as probabilities [B, K, V] (then no draft rows), or null
  float* qxs;          // scratch [rows]: q(x) of each target row's drafted token (with qprob)
  float c2;        // log2(e) / T, the exp2 scale of the streaming pass
  float win;       // top-p candidate window in logit units
  double invT;     // 1 / T in double
  float c2d, wind;  // the same for the draft rows (their own temperature)
  double invTd;
  double top_p;
  ChunkRec* chunk;
  uint32_t* ctop;  // top-k: per (row, chunk), keys of the chunk's CTOP largest thread maxima, descending
  uint64_t* cand;
  RowRec* row;
  int32_t* kidx;
  double* kprob;
  SeqRec* seq;
  uint32_t* seq_cnt;  // per-sequence arrival counters (cleared by the call's streaming kernel)
  uint32_t* smp_cnt;
  int32_t* cflag;     // [1]: ragged offsets valid (written by the streaming kernel)
  double* seg_sum;
  int32_t* seg_last;
  int32_t nitems;  // streaming items (row, chunk): rows * nchunks
  int32_t ulen;   // logits per candidate unit (16-byte vector; 1 on the element-load path)
  UDiv dch;       // division by nchunks
  UDiv drps;      // division by rps
};

// Weight of chunk record (m_c, s_c) in a row whose max is m: the chunk's sum
// of exp((x - m) / T).  The streaming pass sums exp2(x * c2) (c2 = log2(e) / T
// in float) against the integer offset 2^ceil(m_c * c2), or against 2^(m_c * c2)
// itself when that offset overflows float; the record's sum is moved to 2^(m_c *
// c2) by the offset's remainder and then to the row max by exp((m_c - m) / T),
// both in one exp2 of a double exponent.
__device__ __forceinline__ double chunk_weight(double s_c, float m_c, float m, float c2, double invT) {
  if (!(m_c > -INFINITY)) return 0.0;
  const float Mi = __builtin_ceilf(m_c * c2);
  const double f = Mi < INFINITY ? (double)Mi - (double)m_c * (double)c2 : 0.0;
  return s_c * exp2(f + ((double)m_c - (double)m) * (invT * 1.4426950408889634074));
}

// A buffer resource over nbytes at p, for a range every lane of the wave
// shares (a row, or a chunk of one): base and size are read from the first
// lane, so they sit in scalar registers.  Built from a value the compiler
// cannot prove uniform, the resource would be taken lane by lane in a loop
// around every load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* p, int nbytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)(((uint64_t)hi << 32) | lo), (short)0,
                                           __builtin_amdgcn_readfirstlane(nbytes), 0x00020000);
}

// Order-preserving map float -> uint32 (larger float, larger key).
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_val(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
constexpr uint32_t KEY_NEG_INF = 0x007FFFFFu;  // ord_key(-inf)

// A candidate entry as written by the streaming pass (float bits << 32 |
// index) turned into (order key << 32 | index); never 0.
__device__ __forceinline__ uint64_t cand_entry_key(uint64_t raw) {
  return ((uint64_t)ord_key(__uint_as_float((uint32_t)(raw >> 32))) << 32) | (uint32_t)raw;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Logit i of a 16-byte vector of logits (8 bf16 or 4 f32).
template <int DT>
__device__ __forceinline__ float unit_elem(const uint4& r, int i) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  if (DT == D_BF16) return (i & 1) ? bf16_hi(w[i >> 1]) : bf16_lo(w[i >> 1]);
  return __uint_as_float(w[i]);
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* row, int j) {
  if (DT == D_BF16) {
    uint32_t h = *reinterpret_cast<const uint16_t*>(row + (size_t)j * 2);
    return __uint_as_float(h << 16);
  }
  return *reinterpret_cast<const float*>(row + (size_t)j * 4);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_min(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_fmax(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Wave64 reductions with DPP row operations (quad swaps, half-row and row
// mirrors, then row broadcasts 15 and 31); the complete result is in lane 63
// and is returned to every lane through readlane.  Fixed combination order.
template <int CTRL, int RM = 0xF, int BM = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, RM, BM, false);
}
constexpr int DPP_QP_1032 = 0xB1, DPP_QP_2301 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140,
              DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143;
// DPP move whose lanes outside the row mask are left unspecified: the
// reductions below read lane 63 only, which every step writes, and without an
// old value the move folds into the instruction that uses it.
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, RM, 0xF, false);
}

__device__ __forceinline__ uint32_t dpp_wave_umax(uint32_t v) {
  v = max(v, dpp_mov<DPP_QP_1032>(v));
  v = max(v, dpp_mov<DPP_QP_2301>(v));
  v = max(v, dpp_mov<DPP_HALF_MIRROR>(v));
  v = max(v, dpp_mov<DPP_MIRROR>(v));
  v = max(v, dpp_mov<DPP_BCAST15, 0xA>(v));
  v = max(v, dpp_mov<DPP_BCAST31, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Max over the order keys (no NaN canonicalisation, and the integer max folds
// with the DPP moves).
__device__ __forceinline__ float dpp_wave_fmax(float v) { return key_val(dpp_wave_umax(ord_key(v))); }

template <int CTRL, int RM = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_mov<CTRL, RM>((uint32_t)u);
  const uint32_t hi = dpp_mov<CTRL, RM>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ float dpp_wave_fsum(float v) {
  v += __uint_as_float(dpp_mov<DPP_QP_1032>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_QP_2301>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_HALF_MIRROR>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_MIRROR>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_BCAST15, 0xA>(__float_as_uint(v)));
  v += __uint_as_float(dpp_mov<DPP_BCAST31, 0xC>(__float_as_uint(v)));
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(v), 63));
}
__device__ __forceinline__ double dpp_wave_sum(double v) {
  v += dpp_f64<DPP_QP_1032>(v);
  v += dpp_f64<DPP_QP_2301>(v);
  v += dpp_f64<DPP_HALF_MIRROR>(v);
  v += dpp_f64<DPP_MIRROR>(v);
  v += dpp_f64<DPP_BCAST15, 0xA>(v);
  v += dpp_f64<DPP_BCAST31, 0xC>(v);
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Inclusive prefix sums over the 64 lanes of a wave with DPP: shifts of 1, 2,
// 4 and 8 lanes within each row of 16, then the row broadcasts 15 and 31.
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ uint32_t dppz(uint32_t v) {  // 0 where the source lane is outside the row
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, RM, 0xF, false);
}
constexpr int DPP_SHR1 = 0x111, DPP_SHR2 = 0x112, DPP_SHR4 = 0x114, DPP_SHR8 = 0x118;
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t v) {
  v += dppz<DPP_SHR1>(v);
  v += dppz<DPP_SHR2>(v);
  v += dppz<DPP_SHR4>(v);
  v += dppz<DPP_SHR8>(v);
  v += dppz<DPP_BCAST15, 0xA>(v);
  v += dppz<DPP_BCAST31, 0xC>(v);
  return v;
}
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ uint64_t dppz64(uint64_t v) {
  return ((uint64_t)dppz<CTRL, RM>((uint32_t)(v >> 32)) << 32) | dppz<CTRL, RM>((uint32_t)v);
}
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
  v += dppz64<DPP_SHR1>(v);
  v += dppz64<DPP_SHR2>(v);
  v += dppz64<DPP_SHR4>(v);
  v += dppz64<DPP_SHR8>(v);
  v += dppz64<DPP_BCAST15, 0xA>(v);
  v += dppz64<DPP_BCAST31, 0xC>(v);
  return v;
}
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ double dppz_f64(double v) {
  return __longlong_as_double((long long)dppz64<CTRL, RM>((uint64_t)__double_as_longlong(v)));
}
__device__ __forceinline__ double wave_scan_f64(double v) {
  v += dppz_f64<DPP_SHR1>(v);
  v += dppz_f64<DPP_SHR2>(v);
  v += dppz_f64<DPP_SHR4>(v);
  v += dppz_f64<DPP_SHR8>(v);
  v += dppz_f64<DPP_BCAST15, 0xA>(v);
  v += dppz_f64<DPP_BCAST31, 0xC>(v);
  return v;
}
template <typename T>
__device__ __forceinline__ T lane63(T v) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
  }
}

// Block-wide reductions over NW waves (one partial per wave in LDS), fixed
// combination order.
constexpr int MAX_NW = 16;
struct Red {
  double d[MAX_NW];
  float f[MAX_NW];
  int32_t i[MAX_NW];
  uint32_t u[MAX_NW];
};

template <int NW = NWAVE>
__device__ __forceinline__ float block_fmax(float v, Red& r) {
  v = dpp_wave_fmax(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.f[threadIdx.x >> 6] = v;
  __syncthreads();
  float x = r.f[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x = fmaxf(x, r.f[i]);
  return x;
}
template <int NW = NWAVE>
__device__ __forceinline__ double block_sum(double v, Red& r) {
  v = dpp_wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.d[threadIdx.x >> 6] = v;
  __syncthreads();
  double x = r.d[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x += r.d[i];
  return x;
}
template <int NW = NWAVE>
__device__ __forceinline__ int32_t block_min_i(int32_t v, Red& r) {
  v = wave_min(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.i[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t x = r.i[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x = min(x, r.i[i]);
  return x;
}
template <int NW = NWAVE>
__device__ __forceinline__ int32_t block_max_i(int32_t v, Red& r) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.i[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t x = r.i[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x = max(x, r.i[i]);
  return x;
}
template <int NW = NWAVE>
__device__ __forceinline__ uint32_t block_max_u(uint32_t v, Red& r) {
  v = wave_max(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.u[threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t x = r.u[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x = max(x, r.u[i]);
  return x;
}
template <int NW = NWAVE>
__device__ __forceinline__ int32_t block_sum_i(int32_t v, Red& r) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) r.i[threadIdx.x >> 6] = v;
  __syncthreads();
  int32_t x = r.i[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x += r.i[i];
  return x;
}

// Inclusive prefix sum over the block (one value per thread, thread order).
template <int NW = NWAVE>
__device__ __forceinline__ double block_incl_scan(double v, Red& r, double* total) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    double y = __shfl_up(v, o);
    if (l >= o) v += y;
  }
  __syncthreads();
  if (l == 63) r.d[w] = v;
  __syncthreads();
  double off = 0.0;
  for (int i = 0; i < w; ++i) off += r.d[i];
  double tot = r.d[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) tot += r.d[i];
  *total = tot;
  return v + off;
}

// Bitonic sort of n (power of two) 64-bit keys in LDS, descending, by a
// block of BS threads.
template <int BS = WG>
__device__ __forceinline__ void bitonic_desc(uint64_t* a, int n) {
  __syncthreads();
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += BS) {
        int p = i ^ j;
        if (p > i) {
          uint64_t x = a[i], y = a[p];
          bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            a[i] = y;
            a[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Data handed from one workgroup to another within a launch is written and
// read only through these device-scope (agent) relaxed atomics: on gfx950
// they are coherent across the XCDs' separate L2 caches by themselves, so the
// hand-off needs no whole-cache writeback or invalidate (which a device-scope
// fence would issue from every workgroup).
template <typename T>
__device__ __forceinline__ void st_dev(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_dev(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Last-arrival detection for a counter shared by `total` workgroups.  Every
// thread first waits until its own st_dev stores have completed; the barrier
// then orders all of them before thread 0's increment.  The workgroup that
// sees the final count reads the others' records with ld_dev.  The counters
// start every call at zero: the streaming kernel, the call's first launch,
// clears them (clear_counters).
__device__ __forceinline__ bool last_arrival(uint32_t* cnt, uint32_t total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = prev == total - 1;
  }
  __syncthreads();
  return *flag != 0;
}

// The streaming item of this workgroup.  A launch's workgroups go to the
// NXCD XCDs in turn (workgroup i to XCD i mod NXCD); rows are dealt to the
// XCDs in the same turn, so that each XCD streams its rows' chunks in order
// while the XCDs together work on NXCD neighbouring rows at a time: row
// NXCD * (k / nchunks) + (i mod NXCD), chunk k mod nchunks, with k = i / NXCD.
// Measured faster than chunks dealt to the XCDs one by one.  Workgroups past
// the last row (the last turn may be partial) have no item.
constexpr int NXCD = 8;
__device__ __forceinline__ int stream_item(const Args& a) {
  const int i = (int)blockIdx.x;
  const int k = i / NXCD;
  const int r = udiv(k, a.dch);
  return (NXCD * r + i % NXCD) * a.nchunks + (k - r * a.nchunks);
}

// Ragged batches: whether the offsets cu[B + 1] describe a packing of the
// rows (cu[0] = 0, nondecreasing, every K_b <= Kmax, cu[B] = ND), decided
// once per call by the streaming kernel's first workgroup and read by the
// sequence kernel (a.cflag[0]: 1 if they do, 0 if not).
__device__ __forceinline__ void check_offsets(const Args& a) {
  if (!a.cu || blockIdx.x != 0) return;
  bool bad = false;
  for (int s = (int)threadIdx.x; s <= a.B; s += (int)blockDim.x) {
    const int c = a.cu[s];
    const int cn = s < a.B ? a.cu[s + 1] : c;
    bad |= (s == 0 && c != 0) || (s == a.B && c != a.ND) || (s < a.B && (cn < c || cn - c > a.Kmax));
  }
  const int any = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0) a.cflag[0] = any ? 0 : 1;
}

// The arrival counters of the launches that follow, cleared by the call's
// streaming kernel (one per sequence, by workgroup index; its grid has at
// least B workgroups):
// no call depends on what an earlier call left in the scratch.
__device__ __forceinline__ void clear_counters(const Args& a) {
  if (threadIdx.x == 0 && (int)blockIdx.x < a.B) {
    a.seq_cnt[blockIdx.x] = 0u;
    a.smp_cnt[blockIdx.x] = 0u;
  }
}

// Row rl in the order of the packed inputs (every target row, then every
// draft row).  Rectangular: sequence b = rl / rps, its row j = rl - b * rps
// is target row b(K + 1) + j, or draft row NT + bK + (j - K - 1).  Ragged
// batches pass K = 0 and rps = 1, which makes the map the identity.
__device__ __forceinline__ int lin_row(const Args& a, int rl) {
  const int b = udiv(rl, a.drps), j = rl - b * a.rps;
  return b * a.K + j + (j > a.K ? a.NT - a.K - 1 : b);
}

// Temperature-derived scalars of row rl: the draft rows' own (a draft
// sampled at its own temperature is verified against that q), the target's
// for every other row.
struct RowT {
  float c2;     // log2(e) / T
  float win;    // top-p candidate window in logit units
  double invT;  // 1 / T
};
__device__ __forceinline__ RowT row_temp(const Args& a, int rl) {
  return lin_row(a, rl) >= a.NT ? RowT{a.c2d, a.wind, a.invTd} : RowT{a.c2, a.win, a.invT};
}

// Logits of row rl.  The base is chosen by arithmetic on the two pointer
// values: a choice between the two argument fields themselves can be
// compiled into a load from a computed address inside the argument block,
// which moves the whole block to scratch memory.
__device__ __forceinline__ const char* row_ptr(const Args& a, int rl, int esz) {
  const int L = lin_row(a, rl);
  const bool dr = L >= a.NT;
  const size_t idx = (size_t)(dr ? L - a.NT : L);
  const uintptr_t t = (uintptr_t)a.tgt, d = (uintptr_t)a.drf;
  return (const char*)(t + (dr ? d - t : (uintptr_t)0)) + idx * (size_t)a.V * esz;
}

// Batch layouts of the row-merge and sampling kernels.
enum BatchLayout : int {
  LAY_RECT = 0,  // [B, K+1] target and [B, K] draft logit rows
  LAY_RAG = 1,   // ragged: packed rows with offsets cu (a.cu set)
  LAY_QP = 2,    // [B, K+1] target logit rows; q given as probabilities (a.qprob set, no draft rows)
};

// RAG: a ragged batch (a.cu set).
// A sequence: K drafts, its first uniform t0 (= its first target row in
// the packed order), its first drafted token x0 (its draft rows start at
// packed row NT + x0) and, for rectangular batches, its first row s0.
struct SeqGeo {
  int K, t0, x0, s0;
};
template <bool RAG>
__device__ __forceinline__ SeqGeo seq_geo(const Args& a, int b) {
  if (RAG) {
    const int c0 = a.cu[b], c1 = a.cu[b + 1];
    return SeqGeo{c1 - c0, c0 + b, c0, 0};
  }
  return SeqGeo{a.K, b * (a.K + 1), b * a.K, b * a.rps};
}
// Row of the sequence's local row j: 0..K target rows, K+1..2K draft rows.
template <bool RAG>
__device__ __forceinline__ int seq_row(const Args& a, const SeqGeo& g, int j) {
  if (!RAG) return g.s0 + j;
  return j <= g.K ? g.t0 + j : a.NT + g.x0 + (j - g.K - 1);
}

}  // namespace sv

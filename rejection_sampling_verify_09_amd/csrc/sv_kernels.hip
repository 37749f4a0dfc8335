// gfx950 kernels of the speculative-sampling verification step.
//
// The rule (page www.cf-1.com/news/5155685 section 2.2; page
// www.2kiu.com/news/5895634 section 2.2): accept drafted token x_i with
// probability min(1, p_i(x_i)/q_i(x_i)); stop at the first rejection and draw
// its replacement from norm(max(0, p_i - q_i)); after K acceptances draw one
// more token from p_K (the last term of the expected count 1 + a + ... + a^K on
// page www.gsyq.cn/news/428210 section 3.2).  Temperature, top-k and top-p
// act identically on p and q (page www.gsyq.cn/news/428210 section 3.3).
//
// Data flow (one call, all rows of all sequences):
//   stream_kernel   one workgroup per (row, 8192-logit chunk).  Reads the
//                   chunk once from HBM (16-byte non-temporal loads into
//                   registers) and writes the chunk's record: max, sum of
//                   exp((x - max) / T) in the record's convention, the filter
//                   candidates (16-byte units at or above the chunk's bound)
//                   and the greedy arg-max.  Its first workgroups also clear
//                   the call's arrival counters and check ragged offsets.
//   tile_chunk_kernel in the streaming kernel's place when the float32 rows
//                   come from the output projections, whose epilogues
//                   reduced every 64-column tile to a record: the chunk
//                   record from the chunk's 128 tile records, and only the
//                   tiles that reach the candidate bound are read back.
//   seq_kernel      one workgroup per sequence.  One wave merges each row of
//                   the sequence (max, normaliser, top-k / top-p threshold, kept
//                   list in LDS, p or q of the drafted token); a row the
//                   candidate lists cannot decide is merged by the whole
//                   workgroup from the full row.  Then one wave runs the
//                   accept tests, the first-rejection scan and, for filtered
//                   and greedy rows, the final draw from the kept lists.
//   sample_kernel   unfiltered rows only: the final draw needs the whole
//                   residual / bonus row.  One workgroup per (sequence, up to
//                   four 2048-logit chunks) computes the weights in double
//                   and their per-segment sums; the last one to arrive scans
//                   the segment sums, finds the segment holding u*Z and
//                   rescans it.
//   row_kernel      sv_filtered_probs only: the row merges, without
//                   sequences;  probs_kernel then writes full filtered rows.
//   read_kernel     measurement aid (sv_read_floor): a plain read.
#include "sv_common.hpp"

#include <hip/hip_ext.h>

#include <climits>

namespace sv {

constexpr int NCH_LDS = MAX_CHUNKS;  // chunk records of one row held in LDS during its merge
constexpr int ROW_CAND = 1024;       // top-k candidates of one row held in LDS during its merge
constexpr int LOAD_BATCH = 4;        // candidate loads in flight per thread
constexpr int ROW_LOAD_MAX = 4096;   // candidate slots a merge will read before giving up on the lists

// exp(x) in double for the full-row paths: x = (k + 64 i) ln2/64 + r with
// |r| <= ln2/128, exp(x) = 2^i * 2^(k/64) * e^r, the 64 powers 2^(k/64) from a
// table in LDS (built with the library exp2 when such a path starts) and e^r
// from its degree-5 Taylor polynomial (remainder below 4e-17).  Few registers
// and no loop-invariant constants to hoist.
__device__ __forceinline__ double exp_tab(double x, const double* tab) {
  if (!(x > -800.0)) return 0.0;                   // also -inf
  x = x < 800.0 ? x : 800.0;
  const double kf = rint(x * 92.33248261689366);   // 64 / ln2
  // x - kf * ln2/64 with ln2/64 = hi + lo, hi having 22 trailing zero bits
  const double r = fma(kf, -6.619564634077006e-12, fma(kf, -0.01083042468962958, x));
  const double p = fma(fma(fma(fma(fma(r, 1.0 / 120.0, 1.0 / 24.0), r, 1.0 / 6.0), r, 0.5), r, 1.0), r, 1.0);
  const int ki = (int)kf;
  const int j = ki & 63;
  return ldexp(tab[j] * p, (ki - j) >> 6);
}
// 2^(y / 64) in double for y <= 0 (the weights of the unfiltered draw, whose
// exponent, scaling and normaliser fold into y = x * A + B): y = k + f with
// integer k and |f| <= 1/2, 2^(y/64) = 2^(k >> 6) * 2^((k & 63)/64) * e^r with
// r = f ln2/64, |r| <= ln2/128, the powers from the LDS table and e^r from its
// degree-5 Taylor polynomial as in exp_tab.  k is taken by the 1.5 * 2^52
// shift (the sum's low mantissa bits hold round-to-nearest-even of y) and
// 2^(k >> 6) is added to the exponent field, so no conversion or scaling
// instruction is needed.  0 below -64 * 1020 (also -inf), where the result
// would leave the normal range.
__device__ __forceinline__ double exp2_64(double y, const double* tab) {
  if (!(y > -65280.0)) return 0.0;
  const double S = 6755399441055744.0;  // 1.5 * 2^52
  const double ys = y + S;
  const double kf = ys - S;
  const int ki = (int)(uint32_t)__double_as_longlong(ys);
  const double r = (y - kf) * 0.010830424696249145;  // ln2 / 64
  const double p = fma(fma(fma(fma(fma(r, 1.0 / 120.0, 1.0 / 24.0), r, 1.0 / 6.0), r, 0.5), r, 1.0), r, 1.0);
  const double v = tab[ki & 63] * p;
  return __longlong_as_double(__double_as_longlong(v) + ((long long)(ki >> 6) << 52));
}

// chunk_weight with exp2_64 for the power of two (the same value up to a few
// units in the last place).
__device__ __forceinline__ double chunk_weight_tab(double s_c, float m_c, float m, float c2, double invT,
                                                   const double* tab) {
  if (!(m_c > -INFINITY)) return 0.0;
  const float Mi = __builtin_ceilf(m_c * c2);
  const double f = Mi < INFINITY ? (double)Mi - (double)m_c * (double)c2 : 0.0;
  return s_c * exp2_64(64.0 * (f + ((double)m_c - (double)m) * (invT * 1.4426950408889634074)), tab);
}

__device__ __forceinline__ void build_exp_tab(double* tab) {
  __syncthreads();
  if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
  __syncthreads();
}

// The 64 lanes' keys sorted descending across the wave (lane l gets the
// l-th largest): a bitonic network on lane exchanges, no LDS.
__device__ __forceinline__ uint32_t wave_sort_desc(uint32_t key) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const uint32_t other = (uint32_t)__shfl_xor((int)key, j);
      const bool lower = (lane & j) == 0, desc = (lane & k) == 0;
      const uint32_t mx = max(key, other), mn = min(key, other);
      key = (lower == desc) ? mx : mn;
    }
  }
  return key;
}

struct DrawRow {
  double snorm;
  double invT;
  float m;
  uint32_t tau;
  const float* prob;  // a row given as probabilities (then the fields above are unused), or null
};

// Where a merge writes its row's kept list: sink.put(nk, pos, index,
// probability) for each of the nk kept tokens, at its position in ascending
// index order.  Merges of rows that belong to no sequence keep no list.
struct NoSink {
  __device__ __forceinline__ void put(int, int, int32_t, double) const {}
};

constexpr int TK_WAVE_TOP = 16;  // top-k bound: thread maxima each wave posts (k up to NWAVE times this)
struct SmemStream {
  uint64_t cand[NWAVE * CAND_CAP];  // per-wave candidate lists (one flat list after an overflow cut)
  uint64_t tk[WG];
  uint32_t tk16[NWAVE * TK_WAVE_TOP];
  uint32_t tkb;
  uint32_t hist[256];
  int32_t wn[NWAVE];
  float rm[NWAVE];   // per-wave chunk maxima
  float rs[NWAVE];   // per-wave chunk sums (against the wave's offset)
};
struct SmemRow {
  uint64_t keys[KEEP_CAP];
  uint32_t hist[256];
  uint32_t cb[NCH_LDS];
  int32_t cn[NCH_LDS];
  int32_t off[NCH_LDS + 1];
  union {
    struct {  // chunk records, read once at the start of the merge
      double cs[NCH_LDS];
      float cm[NCH_LDS];
      int32_t carg[NCH_LDS];
    };
    uint64_t cand[ROW_CAND];              // top-k candidates at or above the bound
    unsigned long long hist64[256];       // full-row search
  };
};
struct SmemSeq {
  int32_t pidx[KEEP_CAP];
  int32_t qidx[KEEP_CAP];
  double pprob[KEEP_CAP];
  double qprob[KEEP_CAP];
  double px[MAX_RPS];
  int32_t rf[MAX_RPS];
  int32_t nk[MAX_RPS];
  int32_t arg[MAX_RPS];
  int32_t x[MAX_K];
  float u[MAX_K + 1];
};
struct Smem {
  union {
    SmemStream s;
    SmemRow r;
    SmemSeq q;
    double scan[1024];  // one per thread of the largest workgroup (the sequence kernel's)
  };
  Red red;
  DrawRow dr[2];
  double etab[64];  // 2^(j/64) for exp_tab (full-row paths)
  int32_t ncand;
  int32_t flag;
  int32_t i0, i1;
  uint32_t u0;
  float lx;
  double d0;
};

template <int DT>
struct ElemT {
  static constexpr int ESZ = DT == D_BF16 ? 2 : 4;
  static constexpr int EPV = 16 / ESZ;  // logits per 16-byte vector
};

// Local (within-chunk) index of register slot k of thread t.
template <int DT, bool VEC>
__device__ __forceinline__ int local_index(int k, int t) {
  if (VEC) {
    constexpr int EPV = ElemT<DT>::EPV;
    return ((k / EPV) * WG + t) * EPV + (k % EPV);
  }
  return k * WG + t;
}

// Load one chunk into registers: coalesced 16-byte vectors when the row is
// 16-byte aligned, element loads otherwise.  Slots past the row end hold -inf.
template <int DT, bool VEC>
__device__ __forceinline__ void load_chunk(const char* rp, int c0, int cn, float (&v)[EPT]) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x;
  if (VEC) {
    constexpr int EPV = ElemT<DT>::EPV;
    constexpr int NV = EPT / EPV;
    const uint4* p = reinterpret_cast<const uint4*>(rp + (size_t)c0 * ESZ);
    uint4 raw[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int base = (u * WG + t) * EPV;
      if (base < cn) {
        raw[u] = p[u * WG + t];
      } else {
        const uint32_t ninf = DT == D_BF16 ? 0xFF80FF80u : 0xFF800000u;
        raw[u] = make_uint4(ninf, ninf, ninf, ninf);
      }
    }
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
      if (DT == D_BF16) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[u * 8 + 2 * q] = bf16_lo(w[q]);
          v[u * 8 + 2 * q + 1] = bf16_hi(w[q]);
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) v[u * 4 + q] = __uint_as_float(w[q]);
      }
    }
  } else {
    const char* cp = rp + (size_t)c0 * ESZ;
#pragma unroll
    for (int k = 0; k < EPT; ++k) {
      const int l = k * WG + t;
      v[k] = l < cn ? load_elem<DT>(cp, l) : -INFINITY;
    }
  }
}

// Reload register group g (slots 8g..8g+7) of thread t from memory: the chunk
// was just streamed, so this reads L2.  Used for the rare candidate work, so
// that the 32 values need not stay live in registers past the streaming pass.
template <int DT, bool VEC>
__device__ __forceinline__ void load_group(const char* rp, int c0, int cn, int g, float (&w)[8]) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x;
  if (VEC) {
    constexpr int EPV = ElemT<DT>::EPV;
    const uint4* p = reinterpret_cast<const uint4*>(rp + (size_t)c0 * ESZ);
#pragma unroll
    for (int h = 0; h < 8 / EPV; ++h) {
      const int u = g * (8 / EPV) + h;
      const int base = (u * WG + t) * EPV;
      uint4 r = make_uint4(0u, 0u, 0u, 0u);
      if (base < cn) r = p[u * WG + t];
      const uint32_t q[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (DT == D_BF16) {
          w[h * 8 + 2 * e] = base < cn ? bf16_lo(q[e]) : -INFINITY;
          w[h * 8 + 2 * e + 1] = base < cn ? bf16_hi(q[e]) : -INFINITY;
        } else {
          w[h * 4 + e] = base < cn ? __uint_as_float(q[e]) : -INFINITY;
        }
      }
    }
  } else {
    const char* cp = rp + (size_t)c0 * ESZ;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int l = (8 * g + e) * WG + t;
      w[e] = l < cn ? load_elem<DT>(cp, l) : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// row merge helpers
// ---------------------------------------------------------------------------

// Fixed-point scale of probability masses in the full-row search: sums of
// integers are exact in any order, so the search is deterministic.
constexpr double MASS_SCALE = 4503599627370496.0;  // 2^52

// Largest key t >= lo such that F(t) >= target, where F(t) is the number of
// logits of the row with key >= t, or (mass) their probability mass
// exp((x - m) / T) / snorm.  F is non-increasing in t, so t is the key of an
// actual logit: the cut of a top-k (counts) or top-p (mass) set.  Radix
// search, 8 key bits per pass over the whole row (used only when the
// candidate lists cannot decide the cut).
template <int DT, int BS>
__device__ __forceinline__ uint32_t row_radix(const char* rp, int V, uint32_t lo, bool mass, float m, double invT, double snorm,
                              double target, Smem& sm) {
  const int t = threadIdx.x;
  const unsigned long long tgt = mass ? (unsigned long long)(target * MASS_SCALE) : (unsigned long long)target;
  uint32_t prefix = 0, pmask = 0;
  unsigned long long above = 0;  // F of everything in higher bins at the levels fixed so far
  for (int shift = 24; shift >= 0; shift -= 8) {
    __syncthreads();
    for (int d = t; d < 256; d += BS) sm.r.hist64[d] = 0ull;
    __syncthreads();
    for (int j = t; j < V; j += BS) {
      const float x = load_elem<DT>(rp, j);
      const uint32_t key = ord_key(x);
      if (key >= lo && (key & pmask) == prefix) {
        const unsigned long long w =
            mass ? (unsigned long long)(exp_tab(((double)x - (double)m) * invT, sm.etab) / snorm * MASS_SCALE) : 1ull;
        atomicAdd(&sm.r.hist64[(key >> shift) & 255u], w);
      }
    }
    __syncthreads();
    if (t == 0) {
      unsigned long long cum = above;
      int d = 255;
      for (; d > 0; --d) {
        const unsigned long long h = sm.r.hist64[d];
        if (cum + h >= tgt) break;
        cum += h;
      }
      // digits below lo's own digit at this level cannot hold a qualifying key
      sm.i0 = d;
      sm.d0 = __longlong_as_double((long long)cum);
    }
    __syncthreads();
    prefix |= (uint32_t)sm.i0 << shift;
    pmask |= 255u << shift;
    above = (unsigned long long)__double_as_longlong(sm.d0);
  }
  return prefix > lo ? prefix : lo;
}

// One pass over the row for a cut tau: the number of kept logits, their
// normaliser sum exp((x - m) / T), and (when they fit) the kept entries in
// sm.r.keys.
template <int DT, int BS>
__device__ __forceinline__ int row_keep(const char* rp, int V, uint32_t tau, float m, double invT, double* skept, Smem& sm) {
  const int t = threadIdx.x;
  __syncthreads();
  if (t == 0) sm.ncand = 0;
  __syncthreads();
  double acc = 0.0;
  for (int j = t; j < V; j += BS) {
    const float x = load_elem<DT>(rp, j);
    const uint32_t key = ord_key(x);
    if (key >= tau) {
      acc += exp_tab(((double)x - (double)m) * invT, sm.etab);
      const int slot = atomicAdd(&sm.ncand, 1);
      if (slot < KEEP_CAP) sm.r.keys[slot] = ((uint64_t)key << 32) | (uint32_t)j;
    }
  }
  *skept = block_sum<BS / 64>(acc, sm.red);
  return sm.ncand;
}

// The 8 logits j0 .. j0+7 of a row (-inf past V); row and V are the same on
// every lane of the wave.  Rows that are 16-byte aligned with a length of
// whole 16-byte vectors (vec) take one 16-byte buffer load per 8 bf16 (two
// per 8 f32), ranged to the row: a vector past the row end reads as zero
// without a memory access.  No load sits behind a lane condition, so the
// compiler keeps a caller's loads in flight together (plain loads under a
// per-lane bounds branch were each waited for before the next was issued).
template <int DT>
__device__ __forceinline__ void load8(const char* row, int j0, int V, bool vec, float (&x)[8]) {
  if (vec) {
    const __amdgpu_buffer_rsrc_t rs = wave_rsrc(row, V * ElemT<DT>::ESZ);
    if (DT == D_BF16) {
      const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, j0 * 2, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = bf16_lo(w[i]);
        x[2 * i + 1] = bf16_hi(w[i]);
      }
    } else {
      const auto w0 = __builtin_amdgcn_raw_buffer_load_b128(rs, j0 * 4, 0, 0);
      const auto w1 = __builtin_amdgcn_raw_buffer_load_b128(rs, j0 * 4 + 16, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = __uint_as_float(w0[i]);
        x[4 + i] = __uint_as_float(w1[i]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = j0 + e < V ? x[e] : -INFINITY;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = j0 + e < V ? load_elem<DT>(row, j0 + e) : -INFINITY;
  }
}

// load8's vector path split in two, so that a caller can issue every load
// before it unpacks any (the unpacking needs the data, and a wait placed
// before it would hold back the loads behind it).
template <int DT>
struct Raw8 {
  u32x4 w[DT == D_BF16 ? 1 : 2];
};
template <int DT>
__device__ __forceinline__ Raw8<DT> load8_raw(const char* row, int j0, int V) {
  const __amdgpu_buffer_rsrc_t rs = wave_rsrc(row, V * ElemT<DT>::ESZ);
  Raw8<DT> r;
#pragma unroll
  for (int h = 0; h < (DT == D_BF16 ? 1 : 2); ++h) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, j0 * ElemT<DT>::ESZ + 16 * h, 0, 0);
    r.w[h] = u32x4{v[0], v[1], v[2], v[3]};
  }
  return r;
}
template <int DT>
__device__ __forceinline__ void unpack8(const Raw8<DT>& r, int j0, int V, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (DT == D_BF16) {
      x[2 * i] = bf16_lo(r.w[0][i]);
      x[2 * i + 1] = bf16_hi(r.w[0][i]);
    } else {
      x[i] = __uint_as_float(r.w[0][i]);
      x[4 + i] = __uint_as_float(r.w[1][i]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = j0 + e < V ? x[e] : -INFINITY;
}

// Bins of the full-row top-p search: ZB bins per unit of z = (m - x) / T, the
// last bin also holding everything past TOPP_NB / ZB units.  The same f32
// arithmetic in both passes, so an element lands in the same bin each time,
// and bins are monotone in x (a lower bin holds only larger logits).
constexpr int TOPP_NB = 2048;
constexpr float TOPP_ZB = 51.2f;
__device__ __forceinline__ int topp_bin(float x, float m, float itf) {
  const float z = (m - x) * itf;
  return (int)fminf(z * TOPP_ZB, (float)(TOPP_NB - 1));
}

// Top-p cut over the whole row, for rows whose nucleus reaches below the
// candidate window: two pipelined passes instead of row_radix's five
// element-by-element ones.  Pass 1 adds every logit's f32 mass exp(-z) into
// its bin (LDS float atomics) and finds the bin where the cumulative mass
// crosses top_p.  Pass 2 takes, exactly (the fixed-point weights of the wave
// cut, summed as integers), the mass of every logit in the bins above a
// window of five bins around that one, and collects the window's entries;
// they are sorted by key and the cut is the first key at which the mass
// reaches the target, ties included, as in wave_cut64.  Returns false,
// having decided nothing, when the exact cut lies outside the window (the
// f32 masses misplaced it) or the window holds more than ROW_CAND entries;
// the caller then runs row_radix.  Otherwise *tau is the cut, *nall the kept
// count, *skept the sum of exp((x - m) / T) over the kept set and, when
// *nall <= KEEP_CAP, the kept entries (key << 32 | index) are in sm.r.keys.
// Needs sm.etab (build_exp_tab).
template <int DT, int BS>
__device__ __forceinline__ bool row_topp_cut(const char* rp, int V, bool vec, float m, double invT, double snorm,
                                             double top_p, Smem& sm, uint32_t* tau, int* nall, double* skept) {
  static_assert(TOPP_NB % BS == 0 && TOPP_NB * sizeof(float) <= ROW_CAND * sizeof(uint64_t), "histogram layout");
  constexpr int PB = TOPP_NB / BS;  // bins per thread in the scan
  const int t = threadIdx.x;
  const float itf = (float)invT;
  const double A64 = invT * 92.33248261689366;  // 64 log2(e) / T
  float* H = reinterpret_cast<float*>(sm.r.cand);
  __syncthreads();
  for (int d = t; d < TOPP_NB; d += BS) H[d] = 0.0f;
  __syncthreads();
  // pass 1: f32 masses by bin; two tiles of 8 logits per thread in flight
  {
    float xa[8], xb[8];
    int j0 = 8 * t;
    load8<DT>(rp, j0, V, vec, xa);
    for (; j0 < V; j0 += 16 * BS) {
      const int j1 = j0 + 8 * BS;
      load8<DT>(rp, j1, V, vec, xb);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (xa[e] > -INFINITY)
          atomicAdd(&H[topp_bin(xa[e], m, itf)], __builtin_amdgcn_exp2f((xa[e] - m) * itf * 1.44269504f));
      load8<DT>(rp, j1 + 8 * BS, V, vec, xa);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (xb[e] > -INFINITY)
          atomicAdd(&H[topp_bin(xb[e], m, itf)], __builtin_amdgcn_exp2f((xb[e] - m) * itf * 1.44269504f));
    }
  }
  __syncthreads();
  // the bin where the cumulative f32 mass crosses top_p of the total
  double hb[PB], ls = 0.0;
#pragma unroll
  for (int i = 0; i < PB; ++i) {
    hb[i] = (double)H[t * PB + i];
    ls += hb[i];
  }
  double total;
  const double incl = block_incl_scan<BS / 64>(ls, sm.red, &total);
  const double tf = top_p * total;
  int bx = INT_MAX;
  double c = incl - ls;
#pragma unroll
  for (int i = 0; i < PB; ++i) {
    c += hb[i];
    if (bx == INT_MAX && c >= tf) bx = t * PB + i;
  }
  bx = block_min_i<BS / 64>(bx, sm.red);
  if (bx == INT_MAX) bx = TOPP_NB - 1;
  const int bl = max(bx - 2, 0), bh = min(bx + 3, TOPP_NB);
  // pass 2: exact mass above the window, the window's entries
  __syncthreads();
  if (t == 0) {
    sm.ncand = 0;  // kept entries above the window (listed while they fit)
    sm.i1 = 0;     // window entries
  }
  __syncthreads();
  double wa = 0.0, ea = 0.0;  // fixed-point weights (integers, exact as doubles) and exp sums above
  int na = 0;
  {
    float xa[8];
    for (int j0 = 8 * t; j0 < V; j0 += 8 * BS) {
      load8<DT>(rp, j0, V, vec, xa);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = xa[e];
        if (!(x > -INFINITY)) continue;
        const int bin = topp_bin(x, m, itf);
        if (bin >= bh) continue;
        const uint64_t ent = ((uint64_t)ord_key(x) << 32) | (uint32_t)(j0 + e);
        if (bin < bl) {
          const double ew = exp2_64(((double)x - (double)m) * A64, sm.etab);
          wa += (double)(unsigned long long)(ew / snorm * MASS_SCALE);
          ea += ew;
          ++na;
          const int slot = atomicAdd(&sm.ncand, 1);
          if (slot < KEEP_CAP) sm.r.keys[slot] = ent;
        } else {
          const int slot = atomicAdd(&sm.i1, 1);
          if (slot < ROW_CAND) sm.r.cand[slot] = ent;
        }
      }
    }
  }
  const double A = block_sum<BS / 64>(wa, sm.red);
  const double EA = block_sum<BS / 64>(ea, sm.red);
  const int NA = block_sum_i<BS / 64>(na, sm.red);
  const int nw = sm.i1;
  const double tgt = (double)(unsigned long long)(top_p * MASS_SCALE);
  if (nw > ROW_CAND || A >= tgt) return false;  // uniform
  const int np2 = pow2_at_least(nw < 2 ? 2 : nw);
  __syncthreads();
  for (int e = nw + t; e < np2; e += BS) sm.r.cand[e] = 0ull;
  bitonic_desc<BS>(sm.r.cand, np2);
  // the window's weights in key order (contiguous entries per thread)
  constexpr int PW = ROW_CAND / BS;
  uint32_t kw[PW];
  double ww[PW], ew2[PW], lw = 0.0;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int e = t * PW + i;
    const uint64_t en = e < nw ? sm.r.cand[e] : 0ull;
    kw[i] = (uint32_t)(en >> 32);
    ew2[i] = e < nw ? exp2_64(((double)key_val(kw[i]) - (double)m) * A64, sm.etab) : 0.0;
    ww[i] = e < nw ? (double)(unsigned long long)(ew2[i] / snorm * MASS_SCALE) : 0.0;
    lw += ww[i];
  }
  double wtot;
  const double wincl = block_incl_scan<BS / 64>(lw, sm.red, &wtot);
  double cw = A + (wincl - lw);
  int ex = INT_MAX;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    cw += ww[i];
    if (ex == INT_MAX && t * PW + i < nw && cw >= tgt) ex = t * PW + i;
  }
  ex = block_min_i<BS / 64>(ex, sm.red);
  if (ex == INT_MAX) return false;  // the cut lies below the window (uniform)
  __syncthreads();
  const uint32_t tk = (uint32_t)(sm.r.cand[ex] >> 32);
  // kept: everything above the window, and the window's keys >= tk
  int nk = 0;
  double ek = 0.0;
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    if (t * PW + i < nw && kw[i] >= tk) {
      ++nk;
      ek += ew2[i];
    }
  }
  const int NW = block_sum_i<BS / 64>(nk, sm.red);
  const double EW = block_sum<BS / 64>(ek, sm.red);
  const int n = NA + NW;
  if (n <= KEEP_CAP) {
    // the window's kept entries lead the sorted window: append them
    __syncthreads();
    for (int e = t; e < NW; e += BS) sm.r.keys[NA + e] = sm.r.cand[e];
    __syncthreads();
  }
  *tau = tk;
  *nall = n;
  *skept = EA + EW;
  return true;
}

// Radix select (8 bits per pass, counts in LDS) of the k-th largest key among
// the n candidates in sm.r.cand.
template <int BS>
__device__ __forceinline__ uint32_t cand_select(int n, int k, Smem& sm) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    __syncthreads();
    for (int d = t; d < 256; d += BS) sm.r.hist[d] = 0;
    __syncthreads();
    for (int e = t; e < n; e += BS) {
      const uint32_t key = (uint32_t)(sm.r.cand[e] >> 32);
      if ((key & pmask) == prefix) atomicAdd(&sm.r.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (t == 0) {
      int cum = 0, d = 255;
      for (; d > 0; --d) {
        const int h = (int)sm.r.hist[d];
        if (cum + h >= need) break;
        cum += h;
      }
      sm.i0 = d;
      sm.i1 = need - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)sm.i0 << shift;
    pmask |= 255u << shift;
    need = sm.i1;
  }
  return prefix;
}

// Exclusive prefix sum of one int per thread (thread order); *total gets the sum.
template <int NW>
__device__ __forceinline__ int block_excl_scan_i(int v, Red& r, int* total) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (l >= o) x += y;
  }
  __syncthreads();
  if (l == 63) r.i[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
  for (int i = 0; i < w; ++i) off += r.i[i];
#pragma unroll
  for (int i = 0; i < NW; ++i) tot += r.i[i];
  *total = tot;
  return x + off - v;
}

// Sort the first n entries of sm.r.keys descending (pads with zeros).
template <int BS>
__device__ __forceinline__ void sort_keys_desc(int n, Smem& sm) {
  const int np2 = pow2_at_least(n < 2 ? 2 : n);
  __syncthreads();
  for (int e = n + threadIdx.x; e < np2; e += BS) sm.r.keys[e] = 0;
  bitonic_desc<BS>(sm.r.keys, np2);
}

// Top-k / top-p threshold of one row and its kept list.  On entry the chunk
// records are in sm.r (cm, cb, cn) and the row is valid (finite max m;
// for top-p also a finite normaliser rr.S).
template <int DT, int MODE, int BS, class Sink>
__device__ __forceinline__ void filter_row(const Args& a, int rl, const char* rp, float m, RowRec& rr, Smem& sm, const Sink& sink) {
  static_assert(ROW_CAND % BS == 0 && ROW_CAND <= 4 * BS, "top-p scan holds ROW_CAND / BS entries per thread");
  const int t = threadIdx.x, nch = a.nchunks;
  const uint64_t* cand = a.cand + (size_t)rl * nch * CAND_CAP;
  const RowT rt = row_temp(a, rl);
  const double invT = rt.invT;

  // Every finite logit with key >= lo is among the candidates: each chunk
  // emitted all of its finite logits at or above its own bound, and lo is the
  // largest bound (and, for top-p, at least the window below the row max).
  uint32_t lo = block_max_u<BS / 64>(t < nch ? sm.r.cb[t] : 0u, sm.red);
  if (MODE == M_TOPP) lo = max(lo, ord_key(m - rt.win));
  int ncand_total;
  const int my_off = block_excl_scan_i<BS / 64>(t < nch ? sm.r.cn[t] : 0, sm.red, &ncand_total);
  if (t < nch) sm.r.off[t] = my_off;
  if (t == 0) sm.r.off[nch] = ncand_total;
  __syncthreads();

  uint32_t tau = 0;
  int nk = 0;          // kept entries held in sm.r.keys, sorted descending
  bool big = false;    // kept set larger than KEEP_CAP
  double skept = 0.0;  // normaliser over the kept set (when big)
  bool fb = ncand_total > ROW_LOAD_MAX;

  // Top-p whose nucleus reaches below lo takes a second pass with the window
  // doubled (lo2): the lists of the chunks whose own bound lies at or below
  // lo2 hold every unit at or above it, and the few chunks whose bound lies
  // above it (their max is near the row max) are scanned whole.
  const uint32_t lo2 = MODE == M_TOPP ? ord_key(m - 2.0f * rt.win) : lo;
  for (int pass = 0; pass < 2 && !fb; ++pass) {
    const uint32_t lg = pass == 0 ? lo : lo2;
    bool again = false;
    // Candidates at or above lg (at most ROW_CAND), read in batches of
    // LOAD_BATCH loads per thread into sm.r.cand: for the radix select of
    // top-k, for the sort of top-p.
    uint64_t* dstv = sm.r.cand;
    constexpr int cap = ROW_CAND;
    if (t == 0) sm.ncand = 0;
    __syncthreads();
    for (int base = 0; base < ncand_total; base += BS * LOAD_BATCH) {
      uint64_t ck[LOAD_BATCH];
#pragma unroll
      for (int j = 0; j < LOAD_BATCH; ++j) {
        const int e = base + t + j * BS;
        ck[j] = 0ull;
        if (e < ncand_total) {
          int lo_c = 0, hi_c = nch;  // last chunk with off <= e
          while (hi_c - lo_c > 1) {
            const int mid = (lo_c + hi_c) >> 1;
            if (sm.r.off[mid] <= e) lo_c = mid;
            else hi_c = mid;
          }
          // (a chunk whose bound lies above lg is scanned below instead)
          if (sm.r.cb[lo_c] <= lg)
            ck[j] = cand_entry_key(ld_dev(&cand[(size_t)lo_c * CAND_CAP + (e - sm.r.off[lo_c])]));
        }
      }
#pragma unroll
      for (int j = 0; j < LOAD_BATCH; ++j) {
        if (ck[j] != 0ull && (uint32_t)(ck[j] >> 32) >= lg) {
          if (a.ulen > 1) {
            // a candidate unit: its logits at or above lo
            const int st = (int)(uint32_t)ck[j];
            const uint4 r = *reinterpret_cast<const uint4*>(rp + (size_t)st * ElemT<DT>::ESZ);
            for (int i = 0; i < 16 / ElemT<DT>::ESZ; ++i) {
              const float x = unit_elem<DT>(r, i);
              const uint32_t key = ord_key(x);
              if (key >= lg && x > -INFINITY) {
                const int slot = atomicAdd(&sm.ncand, 1);
                if (slot < cap) dstv[slot] = ((uint64_t)key << 32) | (uint32_t)(st + i);
              }
            }
          } else {
            const int slot = atomicAdd(&sm.ncand, 1);
            if (slot < cap) dstv[slot] = ck[j];
          }
        }
      }
    }
    if (pass == 1) {
      for (int c = 0; c < nch; ++c) {
        if (sm.r.cb[c] <= lg) continue;  // uniform
        const int c0 = c * CE, cn = min(CE, a.V - c0);
        const char* cp = rp + (size_t)c0 * ElemT<DT>::ESZ;
        for (int j = 8 * t; j < cn; j += 8 * BS) {
          float x8[8];
          load8<DT>(cp, j, cn, a.ulen > 1, x8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t key = ord_key(x8[e]);
            if (j + e < cn && key >= lg && x8[e] > -INFINITY) {
              const int slot = atomicAdd(&sm.ncand, 1);
              if (slot < cap) dstv[slot] = ((uint64_t)key << 32) | (uint32_t)(c0 + j + e);
            }
          }
        }
      }
    }
    __syncthreads();
    const int cnt = sm.ncand;
    double snorm = rr.S;  // top-p normaliser
    int ns = 0;           // sorted entries available for the top-p walk
    if (cnt > cap) {
      fb = true;
    } else if (MODE == M_TOPK || MODE == M_TOPKP) {
      // fewer than k candidates: with every bound at -inf the row has fewer
      // than k finite logits and all are kept; otherwise the lists cannot decide
      if (cnt < a.top_k && lo > KEY_NEG_INF) fb = true;
      if (!fb) {
        const uint32_t tk = cnt < a.top_k ? KEY_NEG_INF : cand_select<BS>(cnt, a.top_k, sm);
        tau = tk;
        // kept set: candidates with key >= tk, into sm.r.keys
        __syncthreads();
        if (t == 0) sm.i1 = 0;
        __syncthreads();
        double sacc = 0.0;
        for (int e = t; e < cnt; e += BS) {
          const uint64_t ce = sm.r.cand[e];
          const uint32_t key = (uint32_t)(ce >> 32);
          if (key >= tk) {
            sacc += exp(((double)key_val(key) - (double)m) * invT);
            const int slot = atomicAdd(&sm.i1, 1);
            if (slot < KEEP_CAP) sm.r.keys[slot] = ce;
          }
        }
        const double sk = block_sum<BS / 64>(sacc, sm.red);
        const int nall = sm.i1;
        if (nall <= KEEP_CAP) {
          sort_keys_desc<BS>(nall, sm);
          ns = nall;
          nk = nall;
          snorm = sk;
        } else if (MODE == M_TOPK) {
          big = true;
          skept = sk;
        } else {
          fb = true;  // top-p over a top-k set too large for LDS
        }
      }
    } else {  // M_TOPP: every candidate, sorted descending in sm.r.cand
      // Candidates whose mass stays below top_p cannot decide (the nucleus
      // reaches below lg): the next tier is taken without a sort or a walk.
      double ls = 0.0;
      for (int e = t; e < cnt; e += BS)
        ls += exp(((double)key_val((uint32_t)(sm.r.cand[e] >> 32)) - (double)m) * invT);
      if (block_sum<BS / 64>(ls, sm.red) < a.top_p * snorm) {
        (pass == 0 ? again : fb) = true;
      } else {
        const int np2 = pow2_at_least(cnt < 2 ? 2 : cnt);
        __syncthreads();
        for (int e = cnt + t; e < np2; e += BS) sm.r.cand[e] = 0;
        bitonic_desc<BS>(sm.r.cand, np2);
        ns = cnt;
      }
    }
    if (!fb && !again && (MODE == M_TOPP || MODE == M_TOPKP)) {
      // smallest descending prefix whose mass reaches top_p, ties included;
      // thread t holds sorted entries PT t .. PT t + PT - 1
      constexpr int PT = ROW_CAND / BS;
      const uint64_t* srt = MODE == M_TOPP ? sm.r.cand : sm.r.keys;
      uint32_t kv[PT];
      double wv[PT], ls = 0.0;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        const int e = t * PT + i;
        kv[i] = e < ns ? (uint32_t)(srt[e] >> 32) : 0u;
        wv[i] = e < ns ? exp(((double)key_val(kv[i]) - (double)m) * invT) / snorm : 0.0;
        ls += wv[i];
      }
      double tot;
      double C = block_incl_scan<BS / 64>(ls, sm.red, &tot) - ls;
      int first = INT_MAX;
#pragma unroll
      for (int i = 0; i < PT; ++i) {
        C += wv[i];
        if (t * PT + i < ns && C >= a.top_p && first == INT_MAX) first = t * PT + i;
      }
      first = block_min_i<BS / 64>(first, sm.red);
      if (first == INT_MAX) {
        // the nucleus reaches below the candidate window: widen it once
        if (MODE == M_TOPP) (pass == 0 ? again : fb) = true;
        else first = ns - 1;  // round-off kept the top-k mass just below top_p
      }
      if (!fb && !again) {
        if (first < 0) first = 0;
        __syncthreads();
        const uint32_t tp = (uint32_t)(srt[first] >> 32);
        tau = tp > tau ? tp : tau;
        int c = 0;
        double sk = 0.0;
#pragma unroll
        for (int i = 0; i < PT; ++i) {
          const bool kept = t * PT + i < ns && kv[i] >= tau;
          c += kept ? 1 : 0;
          sk += kept ? wv[i] : 0.0;
        }
        nk = block_sum_i<BS / 64>(c, sm.red);
        if (MODE == M_TOPP) {
          // the kept entries lead the sorted candidates
          if (nk <= KEEP_CAP) {
            __syncthreads();
            for (int e = t; e < nk; e += BS) sm.r.keys[e] = sm.r.cand[e];
          } else {
            big = true;
            skept = block_sum<BS / 64>(sk, sm.red) * snorm;
          }
        }
      }
    }
    if (!again) break;
  }

  if (fb) {
    // exact cut by a radix search over the whole row (slow, rare)
    rr.flags |= RF_FALLBACK;
    build_exp_tab(sm.etab);
    uint32_t tk = 0;
    double sk = 0.0;
    if (MODE == M_TOPK || MODE == M_TOPKP) {
      tk = row_radix<DT, BS>(rp, a.V, 0u, false, m, invT, 1.0, (double)a.top_k, sm);
      if (MODE == M_TOPKP) (void)row_keep<DT, BS>(rp, a.V, tk, m, invT, &sk, sm);
    }
    int nall = -1;
    if (MODE == M_TOPP) {
      uint32_t tp;
      int na;
      double sk2;
      if (row_topp_cut<DT, BS>(rp, a.V, a.ulen > 1, m, invT, rr.S, a.top_p, sm, &tp, &na, &sk2)) {
        tau = tp;
        nall = na;
        skept = sk2;
      }
    }
    if (nall < 0) {
      if (MODE == M_TOPP || MODE == M_TOPKP) {
        const double sn = MODE == M_TOPP ? rr.S : sk;
        tau = row_radix<DT, BS>(rp, a.V, tk, true, m, invT, sn, a.top_p, sm);
      } else {
        tau = tk;
      }
      nall = row_keep<DT, BS>(rp, a.V, tau, m, invT, &skept, sm);
    }
    if (nall <= KEEP_CAP) {
      sort_keys_desc<BS>(nall, sm);
      nk = nall;
    } else {
      big = true;
    }
  }

  if (!big) {
    __syncthreads();
    const uint64_t e = t < nk ? sm.r.keys[t] : 0ull;
    const uint32_t key = (uint32_t)(e >> 32);
    const double ex = t < nk ? exp(((double)key_val(key) - (double)m) * invT) : 0.0;
    skept = block_sum<BS / 64>(ex, sm.red);
    // kept list in ascending vocabulary order: re-key as (~index << 32 | key)
    __syncthreads();
    if (t < nk) sm.r.keys[t] = ((uint64_t)(~(uint32_t)e) << 32) | key;
    sort_keys_desc<BS>(nk, sm);
    __syncthreads();
    if (t < nk) {
      const uint64_t f = sm.r.keys[t];
      const float x = key_val((uint32_t)f);
      sink.put(nk, t, (int)~(uint32_t)(f >> 32), exp(((double)x - (double)m) * invT) / skept);
    }
  }
  rr.tau = tau;
  rr.S_kept = skept;
  rr.nkept = big ? -1 : nk;
  if (big) rr.flags |= RF_BIG;
}

__device__ __forceinline__ void store_row(RowRec* p, const RowRec& r) {
  st_dev(&p->S, r.S);
  st_dev(&p->S_kept, r.S_kept);
  st_dev(&p->px, r.px);
  st_dev(&p->m, r.m);
  st_dev(&p->tau, r.tau);
  st_dev(&p->nkept, r.nkept);
  st_dev(&p->flags, r.flags);
  st_dev(&p->arg, r.arg);
}
__device__ __forceinline__ RowRec load_row(const RowRec* p) {
  RowRec r;
  r.S = ld_dev(&p->S);
  r.S_kept = ld_dev(&p->S_kept);
  r.px = ld_dev(&p->px);
  r.m = ld_dev(&p->m);
  r.tau = ld_dev(&p->tau);
  r.nkept = ld_dev(&p->nkept);
  r.flags = ld_dev(&p->flags);
  r.arg = ld_dev(&p->arg);
  r.pad = 0;
  return r;
}

template <int DT, int MODE, int BS, class Sink>
__device__ __forceinline__ RowRec row_finalize(const Args& a, int rl, int xtok, Smem& sm, const Sink& sink) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  constexpr bool FILT = MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP;
  const int t = threadIdx.x, nch = a.nchunks;
  const ChunkRec* cr = a.chunk + (size_t)rl * nch;
  const char* rp = row_ptr(a, rl, ESZ);
  // one round trip: every chunk record, and the logit of the drafted token
  if (t < nch) {
    sm.r.cm[t] = ld_dev(&cr[t].m);
    if (MODE == M_PLAIN || MODE == M_TOPP) sm.r.cs[t] = ld_dev(&cr[t].s);
    if (FILT) {
      sm.r.cb[t] = ld_dev(&cr[t].bound);
      const int nc = ld_dev(&cr[t].ncand);
      sm.r.cn[t] = min(nc, CAND_CAP);
    }
    if (MODE == M_GREEDY) sm.r.carg[t] = ld_dev(&cr[t].arg);
  }
  const bool hx = xtok >= 0 && xtok < a.V;
  if (t == BS - 1) sm.lx = (MODE != M_GREEDY && hx) ? load_elem<DT>(rp, xtok) : -INFINITY;
  __syncthreads();
  const float m = block_fmax<BS / 64>(t < nch ? sm.r.cm[t] : -INFINITY, sm.red);
  RowRec rr;
  rr.S = 0.0;
  rr.S_kept = 0.0;
  rr.px = 0.0;
  rr.m = m;
  rr.tau = 0u;
  rr.nkept = 0;
  rr.flags = 0;
  rr.arg = 0;
  rr.pad = 0;
  bool bad = !(m > -INFINITY && m < INFINITY);
  if (MODE == M_PLAIN || MODE == M_TOPP) {
    const float qm = t < nch ? sm.r.cm[t] : -INFINITY;
    const double s = chunk_weight(sm.r.cs[t], qm, m, row_temp(a, rl).c2, row_temp(a, rl).invT);
    const double S = block_sum<BS / 64>(s, sm.red);
    rr.S = S;
    if (!(S > 0.0 && S < INFINITY)) bad = true;
  }
  if (MODE == M_GREEDY) {
    const int best = block_min_i<BS / 64>((t < nch && sm.r.cm[t] == m) ? sm.r.carg[t] : INT_MAX, sm.red);
    rr.arg = best == INT_MAX ? 0 : best;
  }
  if (FILT) {
    if (!bad) filter_row<DT, MODE, BS>(a, rl, rp, m, rr, sm, sink);
  }
  if (!bad && hx) {
    if (MODE == M_GREEDY) {
      rr.px = xtok == rr.arg ? 1.0 : 0.0;
    } else {
      const float lx = sm.lx;
      if (ord_key(lx) >= rr.tau)
        rr.px = exp(((double)lx - (double)m) * row_temp(a, rl).invT) / (MODE == M_PLAIN ? rr.S : rr.S_kept);
    }
  }
  if (bad) rr.flags |= RF_BAD;
  __syncthreads();
  if (t == 0) store_row(&a.row[rl], rr);
  return rr;
}

// ---------------------------------------------------------------------------
// final draw
// ---------------------------------------------------------------------------

// Probability of token j in a row's kept set (0 outside it).
template <int DT>
__device__ __forceinline__ double kept_prob(const char* rp, int j, const RowRec& R, bool filtered, double invT) {
  const float x = load_elem<DT>(rp, j);
  if (ord_key(x) < R.tau) return 0.0;
  return exp(((double)x - (double)R.m) * invT) / (filtered ? R.S_kept : R.S);
}

// Full-row draw by one workgroup (kept sets too large for a list; an empty
// residual of an unfiltered row).  Tiles of 2048 consecutive logits, 8 per
// thread.  Weights are recomputed rather than held, and the two rows'
// parameters are kept in LDS, so that this rare path stays light on registers
// (it shares a kernel, and so a register allocation, with the streaming pass).
template <int DT>
__device__ __forceinline__ double draw_weight(const char* pr, const char* qr, int j, const DrawRow* dr, bool use_res,
                                              const double* tab) {
  const float xp = load_elem<DT>(pr, j);
  double w = ord_key(xp) >= dr[0].tau ? exp_tab(((double)xp - (double)dr[0].m) * dr[0].invT, tab) / dr[0].snorm : 0.0;
  if (use_res) {
    double q;
    if (dr[1].prob) {
      q = (double)dr[1].prob[j];
    } else {
      const float xq = load_elem<DT>(qr, j);
      q = ord_key(xq) >= dr[1].tau ? exp_tab(((double)xq - (double)dr[1].m) * dr[1].invT, tab) / dr[1].snorm : 0.0;
    }
    const double d = w - q;
    w = d > 0.0 ? d : 0.0;
  }
  return w;
}

template <int DT, int BS>
__device__ __forceinline__ int full_row_sample(const Args& a, double u, const char* pr, const char* qr, bool res, Smem& sm,
                               double* Zout) {
  const int t = threadIdx.x, V = a.V;
  const DrawRow* dr = sm.dr;
  build_exp_tab(sm.etab);
  bool use_res = res;
  double Z = 0.0;
  int lastpos = -1;
  for (int pass = 0; pass < 2; ++pass) {
    Z = 0.0;
    lastpos = -1;
    for (int base = 0; base < V; base += BS * 8) {
      double ts = 0.0;
#pragma unroll 1
      for (int e = 0; e < 8; ++e) {
        const int j = base + t * 8 + e;
        if (j < V) {
          const double w = draw_weight<DT>(pr, qr, j, dr, use_res, sm.etab);
          ts += w;
          if (w > 0.0) lastpos = j;
        }
      }
      Z += block_sum<BS / 64>(ts, sm.red);
    }
    lastpos = block_max_i<BS / 64>(lastpos, sm.red);
    if (!use_res || Z > 0.0) break;
    use_res = false;  // empty residual: draw from p
  }
  const double target = u * Z;
  double run = 0.0;
  int tok = -1;
  for (int base = 0; base < V && tok < 0; base += BS * 8) {
    double ts = 0.0;
#pragma unroll 1
    for (int e = 0; e < 8; ++e) {
      const int j = base + t * 8 + e;
      if (j < V) ts += draw_weight<DT>(pr, qr, j, dr, use_res, sm.etab);
    }
    const double tile = block_sum<BS / 64>(ts, sm.red);
    if (run + tile > target) {
      double tot;
      const double incl = block_incl_scan<BS / 64>(ts, sm.red, &tot);
      __syncthreads();
      sm.scan[t] = incl;
      __syncthreads();
      double C = run + (t > 0 ? sm.scan[t - 1] : 0.0);
      int first = INT_MAX, lastp = -1;
#pragma unroll 1
      for (int e = 0; e < 8; ++e) {
        const int j = base + t * 8 + e;
        if (j < V) {
          const double w = draw_weight<DT>(pr, qr, j, dr, use_res, sm.etab);
          C += w;
          if (w > 0.0) {
            lastp = j;
            if (first == INT_MAX && target < C) first = j;
          }
        }
      }
      first = block_min_i<BS / 64>(first, sm.red);
      tok = first != INT_MAX ? first : block_max_i<BS / 64>(lastp, sm.red);
    }
    run += tile;
  }
  if (tok < 0) tok = lastpos < 0 ? 0 : lastpos;
  *Zout = Z;
  return tok;
}

// Parameters of a row for the full-row draw, into sm.dr[slot].
__device__ __forceinline__ void set_draw_row(const RowRec* r, bool filtered, int slot, double invT, Smem& sm) {
  __syncthreads();
  if (threadIdx.x == 0) {
    sm.dr[slot].invT = invT;
    sm.dr[slot].m = ld_dev(&r->m);
    sm.dr[slot].tau = ld_dev(&r->tau);
    sm.dr[slot].snorm = filtered ? ld_dev(&r->S_kept) : ld_dev(&r->S);
    sm.dr[slot].prob = nullptr;
  }
  __syncthreads();
}

// A row given as probabilities for the full-row draw, into sm.dr[slot].
__device__ __forceinline__ void set_draw_prob_row(const float* prob, int slot, Smem& sm) {
  __syncthreads();
  if (threadIdx.x == 0) sm.dr[slot].prob = prob;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// Candidate units: the filter candidates are taken per unit of contiguous
// logits, the 16 bytes of one vector load (8 bf16 or 4 f32 logits; one logit
// on the element-load path).  A unit is a candidate when its max is at or
// above the chunk's bound, so every logit at or above the bound lies in a
// candidate unit; the row merge reads those units back and keeps their logits
// at or above its own bound.  Register slots u*L .. u*L+L-1 hold unit u.
template <int DT, bool VEC>
struct UnitT {
  static constexpr int L = VEC ? ElemT<DT>::EPV : 1;  // logits per unit
  static constexpr int N = EPT / L;                    // units per thread and chunk
};

// Append every unit of this thread whose max um[u] is at or above thr to its
// wave's candidate list wl and return the wave's count.  Entries are (bits of
// the unit max << 32 | index of its first logit); readers turn the bits into
// an order key (cand_entry_key).  Slots from cap on are dropped (a list of
// 64 * N slots holds every unit of the wave, and then no check is made).
// gm[q] is the max of register slots 8q .. 8q+7: a group with no lane of the
// wave at or above thr costs one compare and one scalar branch.  Called with
// every lane active.
constexpr int FCMP_OGE = 3;  // ordered >= (wave compare mask)
template <int DT, bool VEC>
__device__ __forceinline__ int wave_emit(const float (&um)[UnitT<DT, VEC>::N], const float (&gm)[4], float thr,
                                         int c0, uint64_t* wl, int cap) {
  constexpr int L = UnitT<DT, VEC>::L, UN = UnitT<DT, VEC>::N, UPG = UN / 4;  // units per group of 8 slots
  int wn = 0;
  const int lb = c0 + local_index<DT, VEC>(0, threadIdx.x);  // slot k's index is lb + local_index(k, 0)
  const bool full = UN * 64 <= cap;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (__builtin_amdgcn_fcmpf(gm[q], thr, FCMP_OGE) == 0ull) continue;
#pragma unroll
    for (int i = 0; i < UPG; ++i) {
      const int u = q * UPG + i;
      const bool pr = um[u] >= thr;
      const unsigned long long bm = __builtin_amdgcn_fcmpf(um[u], thr, FCMP_OGE);
      const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)bm, (uint32_t)wn));
      if (pr && (full || pos < cap))
        wl[pos] = ((uint64_t)__float_as_uint(um[u]) << 32) | (uint32_t)(lb + local_index<DT, VEC>(u * L, 0));
      wn += __popcll(bm);
    }
  }
  return wn;
}

// Max without the canonicalisation an IEEE maxnum needs (gfx950
// v_maximum3_f32); logits are never NaN inside the defined input range.
__device__ __forceinline__ float fmax2(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Top-k candidate bound of chunk chunk_id from tm, one group max per thread
// (each the max of disjoint logits of the chunk): the k-th largest of the
// workgroup's group maxima, which is at most the row's k-th largest logit
// (k <= 256; for larger k no bound follows and every finite logit
// qualifies).  Also stores the chunk's CTOP largest group maxima, values of
// the row from which the row merge bounds the row's k-th largest from below.
// Shared memory written here is first written after a barrier of this call.
__device__ __forceinline__ uint32_t chunk_topk_bound(const Args& a, int chunk_id, float tm, Smem& sm) {
  const int t = threadIdx.x;
  if (a.top_k <= NWAVE * TK_WAVE_TOP) {
    // k <= 64: each wave sorts its 64 group maxima in registers and posts
    // its 16 largest; wave 0 sorts those 64.  Their k-th largest is at most
    // the k-th largest of all 256 group maxima (a subset's), so at least
    // k logits of the row lie at or above it, and it equals it whenever no
    // wave holds more than 16 of the chunk's k largest; their 8 largest
    // are the chunk's 8 largest group maxima (each wave posted its own 8).
    // Two barriers instead of the sorting network's 36.
    const int lane = t & 63, w = t >> 6;
    const uint32_t kw = wave_sort_desc(ord_key(tm));
    if (lane < TK_WAVE_TOP) sm.s.tk16[w * TK_WAVE_TOP + lane] = kw;
    __syncthreads();
    if (t < 64) {
      const uint32_t k2 = wave_sort_desc(sm.s.tk16[lane]);
      if (lane == a.top_k - 1) sm.s.tkb = k2;
      if (lane < CTOP) __builtin_nontemporal_store(k2, &a.ctop[(size_t)chunk_id * CTOP + lane]);
    }
    __syncthreads();
    return sm.s.tkb;
  }
  __syncthreads();
  sm.s.tk[t] = ord_key(tm);
  bitonic_desc(sm.s.tk, WG);
  const uint32_t bound = a.top_k <= WG ? (uint32_t)sm.s.tk[a.top_k - 1] : KEY_NEG_INF;
  if (t < CTOP) __builtin_nontemporal_store((uint32_t)sm.s.tk[t], &a.ctop[(size_t)chunk_id * CTOP + t]);
  return bound;
}

// Candidate emission and the chunk record, once the chunk max mc (and for
// sum modes the chunk sum s in the record's convention, chunk_weight; in
// greedy mode the arg-max) and, for filtered modes, the candidate bound are
// known.  um / gm are the unit and group maxima of this thread.  Shared
// memory written here is first written after a barrier of this call, so a
// workgroup can run it for consecutive items without a barrier in between.
// Only the next launch reads what is stored here, so no atomic or fence is
// needed; the stores are nontemporal, so that the records and lists do not
// sit dirty in this launch's cache.
template <int DT, int MODE, bool VEC>
__device__ __forceinline__ void chunk_lists(const Args& a, int item, const float (&um)[UnitT<DT, VEC>::N],
                                            const float (&gm)[4], float mc, double s, int arg, uint32_t bound,
                                            Smem& sm) {
  constexpr bool FILT = MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP;
  constexpr int UL = UnitT<DT, VEC>::L, UN = UnitT<DT, VEC>::N;
  const int t = threadIdx.x;
  const int rl = udiv(item, a.dch);
  const int c0 = (item - rl * a.nchunks) * CE;
  const int chunk_id = item;
  int nc = 0;
  if (FILT) {
    const float thr = bound > KEY_NEG_INF ? key_val(bound) : -3.402823466e38f;
    const int w = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wn = wave_emit<DT, VEC>(um, gm, thr, c0, &sm.s.cand[w * CAND_CAP], CAND_CAP);
    if ((t & 63) == 0) sm.s.wn[w] = wn;
    __syncthreads();
    const int n0 = sm.s.wn[0], n1 = sm.s.wn[1], n2 = sm.s.wn[2], n3 = sm.s.wn[3];
    nc = (n0 + n1) + (n2 + n3);
    uint64_t* dst = a.cand + (size_t)chunk_id * CAND_CAP;
    if (nc <= CAND_CAP) {
      const int off = (w > 0 ? n0 : 0) + (w > 1 ? n1 : 0) + (w > 2 ? n2 : 0);
      for (int j = t & 63; j < wn; j += 64) __builtin_nontemporal_store(sm.s.cand[w * CAND_CAP + j], &dst[off + j]);
    } else {
      // Too many: keep exactly the units above the (CAND_CAP+1)-th largest
      // unit max (radix select over the registers) and raise the bound to match.
      uint32_t prefix = 0, pmask = 0;
      int need = CAND_CAP + 1;
      for (int shift = 24; shift >= 0; shift -= 8) {
        __syncthreads();
        sm.s.hist[t] = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const uint32_t key = ord_key(um[u]);
          if (um[u] >= thr && (key & pmask) == prefix) atomicAdd(&sm.s.hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (t == 0) {
          int cum = 0, d = 255;
          for (; d > 0; --d) {
            const int h = (int)sm.s.hist[d];
            if (cum + h >= need) break;
            cum += h;
          }
          sm.i0 = d;
          sm.i1 = need - cum;
          sm.ncand = 0;
        }
        __syncthreads();
        prefix |= (uint32_t)sm.i0 << shift;
        pmask |= 255u << shift;
        need = sm.i1;
      }
      bound = prefix + 1u;  // every unit with max key >= bound fits
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        if (um[u] >= thr && ord_key(um[u]) >= bound) {
          const int s2 = atomicAdd(&sm.ncand, 1);
          if (s2 < CAND_CAP)
            sm.s.cand[s2] = ((uint64_t)__float_as_uint(um[u]) << 32) | (uint32_t)(c0 + local_index<DT, VEC>(u * UL, t));
        }
      }
      __syncthreads();
      nc = sm.ncand;
      for (int j = t; j < nc; j += WG) __builtin_nontemporal_store(sm.s.cand[j], &dst[j]);
    }
  }
  if (t == 0) {
    // the record as two 16-byte stores that do not stay in this cache (only
    // the next launch reads them)
    u32x4* rp4 = reinterpret_cast<u32x4*>(&a.chunk[chunk_id]);
    const uint64_t sb = (uint64_t)__double_as_longlong(s);
    __builtin_nontemporal_store(u32x4{(uint32_t)sb, (uint32_t)(sb >> 32), __float_as_uint(mc), bound}, rp4);
    __builtin_nontemporal_store(u32x4{(uint32_t)nc, (uint32_t)arg, 0u, 0u}, rp4 + 1);
  }
}

// The streaming kernel's candidate bound (top-p: the window below the chunk
// max, which is <= the row max; top-k: chunk_topk_bound over the thread
// maxima tm), then the lists and the record.
template <int DT, int MODE, bool VEC>
__device__ __forceinline__ void stream_emit(const Args& a, int item, const float (&um)[UnitT<DT, VEC>::N],
                                            const float (&gm)[4], float tm, float mc, double s, int arg,
                                            Smem& sm) {
  constexpr bool FILT = MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP;
  uint32_t bound = 0u;
  if (FILT) {
    const int rl = udiv(item, a.dch);
    bound = MODE == M_TOPP ? ord_key(mc - row_temp(a, rl).win) : chunk_topk_bound(a, item, tm, sm);
  }
  chunk_lists<DT, MODE, VEC>(a, item, um, gm, mc, s, arg, bound, sm);
}

// Element-load path (rows not 16-byte aligned): one workgroup per (row,
// chunk).  No workgroup waits on another: the row merge runs in the next
// launch.
template <int DT, int MODE>
__global__ void __launch_bounds__(WG, (stream_wg_per_cu<DT, false>())) stream_kernel_elem(Args a) {
  __shared__ Smem sm;
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x;
  clear_counters(a);
  check_offsets(a);
  const int item = stream_item(a);
  if (item >= a.nitems) return;
  const int rl = udiv(item, a.dch);
  const int c0 = (item - rl * a.nchunks) * CE;
  const int cn = min(CE, a.V - c0);
  const char* rp = row_ptr(a, rl, ESZ);
  float v[EPT];
  load_chunk<DT, false>(rp, c0, cn, v);
  // units are single logits here: the unit maxima are v itself
  float gm[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float x = v[8 * g];
#pragma unroll
    for (int i = 1; i < 8; ++i) x = fmax2(x, v[8 * g + i]);
    gm[g] = x;
  }
  const float tm = fmax2(fmax2(gm[0], gm[1]), fmax2(gm[2], gm[3]));
  const float mc = block_fmax(tm, sm.red);
  double s = 0.0;
  if (MODE == M_PLAIN || MODE == M_TOPP) {
    // in the record's convention (chunk_weight)
    double acc = 0.0;
    if (mc > -INFINITY) {
      const float c2f = row_temp(a, rl).c2;
      const double c2 = (double)c2f;
      const float Mi = __builtin_ceilf(mc * c2f);
      const double off = Mi < INFINITY ? (double)Mi : (double)mc * c2;
#pragma unroll
      for (int k = 0; k < EPT; ++k)
        if (v[k] > -INFINITY) acc += exp2((double)v[k] * c2 - off);
    }
    s = block_sum(acc, sm.red);
  }
  int arg = 0;
  if (MODE == M_GREEDY) {
    int best = INT_MAX;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (v[k] == mc) best = min(best, k * WG + t);
    best = block_min_i(best, sm.red);
    arg = c0 + (best == INT_MAX ? 0 : best);
  }
  stream_emit<DT, MODE, false>(a, item, v, gm, tm, mc, s, arg, sm);
}

// 16-byte vectors of one chunk per thread (thread t, vector u holds the
// chunk's vector u*WG + t).
template <int DT>
struct ChunkRaw {
  uint4 r[EPT / ElemT<DT>::EPV];
};

// Cache policy of the streaming loads: non-temporal (the logits are read
// once; measured 7% faster than the default policy for a plain read).
constexpr int CPOL_NT = 2;

// Issue the loads of the chunk of row rl at logit c0 (cn logits) as buffer
// loads whose range ends with the chunk: a vector past the row end reads as
// zero without a memory access, so no load depends on a lane condition.
// Vector u of the threads has its own descriptor, based at the chunk's byte
// u*WG*16 and sized to what is left of the chunk, so that the range check
// sees the whole offset (the lane offset t*16 is the only offset of the load).
template <int DT>
__device__ __forceinline__ void issue_chunk(const Args& a, int rl, int c0, int cn, ChunkRaw<DT>& cr) {
  constexpr int ESZ = ElemT<DT>::ESZ, NV = EPT / ElemT<DT>::EPV;
  const char* cp = row_ptr(a, rl, ESZ) + (size_t)c0 * ESZ;
  const int nbytes = cn * ESZ;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int ub = u * WG * 16;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cp + ub), (short)0, max(nbytes - ub, 0), 0x00020000);
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)threadIdx.x * 16, 0, CPOL_NT);
    cr.r[u] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Widen 16-byte vector r into its EPV logits.
template <int DT>
__device__ __forceinline__ void unpack16(const uint4& r, float* v) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (DT == D_BF16) {
      v[2 * q] = bf16_lo(w[q]);
      v[2 * q + 1] = bf16_hi(w[q]);
    } else {
      v[q] = __uint_as_float(w[q]);
    }
  }
}

// Sum over chunk logits cp[0 .. cn) of exp2((x - mc) * c2) in double, this
// thread's share (strided by the workgroup).  Used only when mc * c2
// overflows float; kept out of line so that its constants do not occupy
// registers in the streaming loop.
template <int DT>
__device__ __noinline__ double chunk_sum_slow(const char* cp, int cn, float mc, float c2) {
  double d = 0.0;
  for (int l = threadIdx.x; l < cn; l += WG) {
    const double x = (double)load_elem<DT>(cp, l);
    if (x > -INFINITY) d += exp2((x - (double)mc) * (double)c2);
  }
  return d;
}

// Vector path: one workgroup per (row, chunk), loading through buffer loads
// (issue_chunk).  The exp sum of each wave is taken against the integer
// offset Mw = ceil(mw * c2) of its max mw (so every term is exp2 of at most a
// fraction above 0), and the wave sums meet at the chunk's offset
// Mi = ceil(mc * c2) by exact ldexp (offsets far apart scale a term to zero
// either way): that is the record's convention (chunk_weight), reached with
// one barrier for the chunk max and sum together.  Only when mc * c2
// overflows float is the chunk summed again, in double, from memory.  No
// workgroup waits on another: the row merge runs in the next launch.
template <int DT, int MODE>
__device__ __forceinline__ void stream_vec_body(const Args& a, int item, int rl, int c0, int cn,
                                                const ChunkRaw<DT>& cr, Smem& sm) {
  constexpr int EPV = ElemT<DT>::EPV, NV = EPT / EPV;
  constexpr bool SUM = MODE == M_PLAIN || MODE == M_TOPP;
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const float c2 = row_temp(a, rl).c2;

  float v[EPT], um[NV];
  const int nvec = cn / EPV;  // vectors in the chunk (the row's last chunk has fewer than WG * NV)
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    unpack16<DT>(cr.r[u], &v[u * EPV]);
    if (nvec < WG * NV) {
      const bool out = t >= nvec - u * WG;  // vector u*WG + t lies past the row end (it read as zero)
#pragma unroll
      for (int e = 0; e < EPV; ++e) v[u * EPV + e] = out ? -INFINITY : v[u * EPV + e];
    }
    float x = v[u * EPV];
#pragma unroll
    for (int e = 1; e < EPV; ++e) x = fmax2(x, v[u * EPV + e]);
    um[u] = x;
  }
  float gm[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    constexpr int UPG = NV / 4;
    float x = um[g * UPG];
#pragma unroll
    for (int i = 1; i < UPG; ++i) x = fmax2(x, um[g * UPG + i]);
    gm[g] = x;
  }
  const float tm = fmax2(fmax2(gm[0], gm[1]), fmax2(gm[2], gm[3]));

  // chunk max and sum: one wave-level pass each, one barrier.  The terms are
  // taken against the wave's offset Mw (-1e30 for an all -inf wave: its terms
  // are 0) and summed pairwise.
  const float mw = dpp_wave_fmax(tm);
  if (SUM) {
    const float Mw = fmax2(__builtin_ceilf(mw * c2), -1.0e30f);
    float e[EPT];
#pragma unroll
    for (int k = 0; k < EPT; ++k) e[k] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[k], c2, -Mw));
#pragma unroll
    for (int h = 1; h < EPT; h *= 2) {
#pragma unroll
      for (int k = 0; k < EPT; k += 2 * h) e[k] += e[k + h];
    }
    const float sw = dpp_wave_fsum(e[0]);
    if ((t & 63) == 0) sm.s.rs[w] = sw;
  }
  if ((t & 63) == 0) sm.s.rm[w] = mw;
  __syncthreads();
  float mc = sm.s.rm[0];
#pragma unroll
  for (int i = 1; i < NWAVE; ++i) mc = fmax2(mc, sm.s.rm[i]);
  double s = 0.0;  // the record's sum: thread 0 stores it
  if (SUM && mc > -INFINITY) {
    const float Mi = __builtin_ceilf(mc * c2);
    if (Mi < INFINITY) {
      if (w == 0) {
#pragma unroll
        for (int i = 0; i < NWAVE; ++i) {
          const float m = sm.s.rm[i];
          if (m > -INFINITY)
            s += __builtin_amdgcn_ldexp((double)sm.s.rs[i], (int)fmaxf(__builtin_ceilf(m * c2) - Mi, -2048.0f));
        }
      }
    } else {
      constexpr int ESZ = ElemT<DT>::ESZ;
      s = block_sum(chunk_sum_slow<DT>(row_ptr(a, rl, ESZ) + (size_t)c0 * ESZ, cn, mc, c2), sm.red);
    }
  }

  int arg = 0;
  if (MODE == M_GREEDY) {
    int best = INT_MAX;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (v[k] == mc) best = min(best, local_index<DT, true>(k, t));
    best = block_min_i(best, sm.red);
    arg = c0 + (best == INT_MAX ? 0 : best);
  }
  stream_emit<DT, MODE, true>(a, item, um, gm, tm, mc, s, arg, sm);
}

template <int DT, int MODE>
__global__ void __launch_bounds__(WG, (stream_wg_per_cu<DT, true>())) stream_kernel_vec(Args a) {
  __shared__ Smem sm;
  // The chunk's loads go out first, before the per-call bookkeeping: a
  // workgroup past the last item (idle) addresses item 0 with an empty range,
  // so its loads touch no memory, and leaves after the bookkeeping (the first
  // workgroup, which checks the offsets, is never idle).
  const int it = stream_item(a);
  const bool idle = it >= a.nitems;
  const int item = idle ? 0 : it;
  const int rl = udiv(item, a.dch);
  const int c0 = (item - rl * a.nchunks) * CE;
  const int cn = idle ? 0 : min(CE, a.V - c0);
  ChunkRaw<DT> cr;
  issue_chunk<DT>(a, rl, c0, cn, cr);
  clear_counters(a);
  check_offsets(a);
  if (idle) return;
  stream_vec_body<DT, MODE>(a, item, rl, c0, cn, cr, sm);
}

// ---------------------------------------------------------------------------
// chunk records from the output projections' tile statistics
// ---------------------------------------------------------------------------

// In place of the streaming kernel when the float32 logit rows were written
// by the output projections together with their tile statistics (TS_SUM or
// TS_ARG records of TILE_N-column tiles in R, whose rows number rstride, of
// ntg tiles per row).  One workgroup per (row, chunk) item, as there.  The
// chunk's record follows from its 128 tiles': the max is the largest tile
// max; the sum is the tiles' sums moved from their offsets ceil(max_t * c2)
// to the chunk's ceil(mc * c2) by exact ldexp (the record's convention,
// chunk_weight); the greedy arg-max is the lowest arg-max among the tiles
// holding mc.  Filtered rows read back only the tiles whose max reaches the
// chunk's candidate bound (no unit of another tile can reach it), with the
// top-k bound taken over the tile maxima, and emit those units as the
// streaming kernel does.  When mc * c2 overflows float the sum is taken from
// the logits, as there.
template <int MODE>
__global__ void __launch_bounds__(WG, (stream_wg_per_cu<D_F32, true>()))
    tile_chunk_kernel(Args a, const uint2* __restrict__ R, int rstride, int ntg) {
  constexpr bool FILT = MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP;
  constexpr bool SUM = MODE == M_PLAIN || MODE == M_TOPP;
  constexpr int EPV = ElemT<D_F32>::EPV, NV = EPT / EPV;
  __shared__ Smem sm;
  __shared__ float tmx[TILES_PER_CHUNK];  // the chunk's tile maxima
  const int item = stream_item(a);
  clear_counters(a);
  check_offsets(a);
  if (item >= a.nitems) return;
  const int rl = udiv(item, a.dch);
  const int c0 = (item - rl * a.nchunks) * CE;
  const int cn = min(CE, a.V - c0);
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const RowT rt = row_temp(a, rl);

  // thread t < 128: tile c0 / TILE_N + t
  const int g = c0 / TILE_N + t;
  const bool has = t < TILES_PER_CHUNK && g < ntg;
  float tmax = -INFINITY;
  uint32_t tv = 0u;
  if (has) {
    const uint2 r = R[((size_t)(g / TILE_GROUP) * rstride + lin_row(a, rl)) * TILE_GROUP + g % TILE_GROUP];
    tmax = __uint_as_float(r.x);
    tv = r.y;
  }
  if (FILT && t < TILES_PER_CHUNK) tmx[t] = tmax;
  const float mw = dpp_wave_fmax(tmax);
  if ((t & 63) == 0) sm.s.rm[w] = mw;
  __syncthreads();
  float mc = sm.s.rm[0];
#pragma unroll
  for (int i = 1; i < NWAVE; ++i) mc = fmax2(mc, sm.s.rm[i]);

  double s = 0.0;
  if (SUM && mc > -INFINITY) {
    const float Mi = __builtin_ceilf(mc * rt.c2);
    if (Mi < INFINITY) {
      double term = 0.0;
      if (tmax > -INFINITY)
        term = __builtin_amdgcn_ldexp((double)__uint_as_float(tv),
                                      (int)fmaxf(__builtin_ceilf(tmax * rt.c2) - Mi, -2048.0f));
      s = block_sum(term, sm.red);
    } else {
      s = block_sum(chunk_sum_slow<D_F32>(row_ptr(a, rl, 4) + (size_t)c0 * 4, cn, mc, rt.c2), sm.red);
    }
  }
  int arg = 0;
  if (MODE == M_GREEDY) {
    const int best = block_min_i(has && tmax == mc ? (int)tv : INT_MAX, sm.red);
    arg = best == INT_MAX ? c0 : best;
  }

  float um[NV], gm[4];
#pragma unroll
  for (int u = 0; u < NV; ++u) um[u] = -INFINITY;
  uint32_t bound = 0u;
  if (FILT) {
    bound = MODE == M_TOPP ? ord_key(mc - rt.win) : chunk_topk_bound(a, item, tmax, sm);
    const float thr = bound > KEY_NEG_INF ? key_val(bound) : -3.402823466e38f;
    // Vector u * WG + t of the chunk (logits 4 (u * WG + t) .. + 3) lies in
    // tile 16 u + t / 16.  A vector of a tile below thr addresses the end of
    // its descriptor's range instead: it reads as zero and touches no memory.
    const char* cp = row_ptr(a, rl, 4) + (size_t)c0 * 4;
    const int nbytes = cn * 4;
    uint4 raw[NV];
    bool rd[NV];
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      const int ub = u * WG * 16;
      const int nrec = max(nbytes - ub, 0);
      const __amdgpu_buffer_rsrc_t rs =
          __builtin_amdgcn_make_buffer_rsrc((void*)(cp + ub), (short)0, nrec, 0x00020000);
      rd[u] = tmx[(WG * EPV / TILE_N) * u + t / (TILE_N / EPV)] >= thr;
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, rd[u] ? t * 16 : nrec, 0, CPOL_NT);
      raw[u] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    const int nvec = cn / EPV;
#pragma unroll
    for (int u = 0; u < NV; ++u) {
      float v[EPV];
      unpack16<D_F32>(raw[u], v);
      const bool out = !rd[u] || t >= nvec - u * WG;
      float x = v[0];
#pragma unroll
      for (int e = 1; e < EPV; ++e) x = fmax2(x, v[e]);
      um[u] = out ? -INFINITY : x;
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) gm[q] = fmax2(um[2 * q], um[2 * q + 1]);
  chunk_lists<D_F32, MODE, true>(a, item, um, gm, mc, s, arg, bound, sm);
}

// ---------------------------------------------------------------------------
// row merges: one wave per row (wave_row), the whole workgroup when the
// candidate lists cannot decide (row_finalize)
// ---------------------------------------------------------------------------

// Orders LDS accesses of the lanes of one wave (the wave's LDS operations
// execute in order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T>
__device__ __forceinline__ T lane_bcast(T v, int lane) {
  return __shfl(v, lane);
}

// Appends each lane's entries vals[i] with pred[i] to the wave's list
// (lane-major order) after the n entries already there; entries from cap on
// are dropped.  Returns the new count.  One prefix sum over the lanes' counts
// instead of a ballot per entry, so the entries are independent work.
template <int N>
__device__ __forceinline__ int wave_append(const uint64_t (&vals)[N], const bool (&pred)[N], uint64_t* list, int n,
                                           int cap) {
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) cnt += pred[i] ? 1u : 0u;
  const uint32_t incl = wave_scan_u32(cnt);
  int pos = n + (int)(incl - cnt);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (pred[i] && pos < cap) list[pos] = vals[i];
    pos += pred[i] ? 1 : 0;
  }
  return n + (int)lane63(incl);
}

constexpr int WR_EPL = KEEP_CAP / 64;  // candidate entries per lane in a wave merge
constexpr int WR_LOADS = 16;           // candidate loads per lane in one round trip
constexpr int WR_ITER = 32;            // distinct keys the descending walk takes before the radix search

struct WaveRowSm {
  union {
    uint64_t keys[KEEP_CAP];       // candidates at or above lo (ord_key << 32 | index)
    unsigned long long hist[256];  // radix-select bins
    int32_t kept[KEEP_CAP];        // kept indices (for their ascending order)
    struct {                       // rank cut of at most 64 entries
      uint32_t k[64], ks[64];
      unsigned long long ws[64];
    } cut;
  };
};

// Largest key t among the wave's entries (key ek, weight wt; weight 0 = no
// entry) whose weight at or above t, F(t), reaches target: the cut of a
// top-k set (weights 1) or a top-p set (weights the probability in fixed
// point).  F is non-increasing in t, so the result is the key of an entry.
// Returns 0 when the total weight is below target.  Radix search over the
// key, 8 bits per pass, bins in LDS.
template <int S = WR_EPL>
__device__ __forceinline__ uint32_t wave_radix(const uint32_t (&ek)[S], const unsigned long long (&wt)[S],
                               unsigned long long target, unsigned long long* hist) {
  const int lane = threadIdx.x & 63;
  unsigned long long tot = 0;
#pragma unroll
  for (int r = 0; r < S; ++r) tot += wt[r];
  tot = lane63(wave_scan_u64(tot));
  if (tot < target) return 0u;
  uint32_t prefix = 0, pmask = 0;
  unsigned long long above = 0;  // F of everything in higher bins at the levels fixed so far
  for (int shift = 24; shift >= 0; shift -= 8) {
    wave_sync();
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[lane * 4 + q] = 0ull;
    wave_sync();
#pragma unroll
    for (int r = 0; r < S; ++r)
      if (wt[r] != 0ull && (ek[r] & pmask) == prefix) atomicAdd(&hist[(ek[r] >> shift) & 255u], wt[r]);
    wave_sync();
    // lane L holds digits 255 - 4L - q (descending digit order across the wave)
    unsigned long long h[4], ls = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = hist[255 - 4 * lane - q];
      ls += h[q];
    }
    const unsigned long long ex = above + wave_scan_u64(ls) - ls;
    const bool cross = ex < target && ex + ls >= target;
    const unsigned long long bm = __ballot(cross);
    const int src = bm ? __ffsll((unsigned long long)bm) - 1 : 63;
    int d = 0;
    unsigned long long na = ex;
    if (cross) {
      unsigned long long c = ex;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (c + h[q] >= target) {
          d = 255 - 4 * lane - q;
          na = c;
          break;
        }
        c += h[q];
      }
    }
    d = lane_bcast(d, src);
    na = lane_bcast(na, src);
    prefix |= (uint32_t)d << shift;
    pmask |= 255u << shift;
    above = na;
  }
  return prefix;
}

// Descending walk over the distinct keys of the wave's entries in slots
// 0..S-1 (key ek, 0 for none; fixed-point weight wt, equal for equal keys):
// returns the first key at which the running weight reaches target, 0 when
// the entries run out first, or 1 (not the key of any finite logit) when
// WR_ITER keys were not enough; the caller then uses the radix search.  The
// same cut as wave_radix, cheap when it lies within the first few keys, as a
// nucleus usually does.
template <int S>
__device__ __forceinline__ uint32_t wave_walk(const uint32_t (&ek)[WR_EPL], const unsigned long long (&wt)[WR_EPL],
                                              unsigned long long target) {
  unsigned long long run = 0;
  uint32_t hi = 0xFFFFFFFFu;
  for (int it = 0; it < WR_ITER; ++it) {
    uint32_t lm = 0;
#pragma unroll
    for (int r = 0; r < S; ++r)
      if (ek[r] < hi && ek[r] > lm) lm = ek[r];
    const uint32_t km = dpp_wave_umax(lm);
    if (km == 0u) return 0u;
    int cnt = 0, src = -1;
    unsigned long long wsel = 0;
#pragma unroll
    for (int r = 0; r < S; ++r) {
      const unsigned long long bm = __ballot(ek[r] == km);
      cnt += __popcll(bm);
      if (src < 0 && bm != 0ull) {  // uniform: the first slot holding the key
        src = __ffsll(bm) - 1;
        wsel = wt[r];
      }
    }
    const unsigned long long w = ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(wsel >> 32), src) << 32) |
                                 (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)wsel, src);
    run += (unsigned long long)cnt * w;
    if (run >= target) return km;
    hi = km;
  }
  return 1u;
}

// The same cut as wave_radix for at most n <= 64 entries, one per lane (key k,
// 0 for none; weight wt): each entry's stable rank in descending key order
// (one pass over the n keys), the weights in that order, one prefix
// sum, and the key at the first position where it reaches target.  The
// weights of a key's ties all precede the next smaller key, so that key is
// the largest t whose weight at or above t reaches target.
__device__ __forceinline__ uint32_t wave_cut64(uint32_t k, unsigned long long wt, unsigned long long target, int n,
                                               WaveRowSm& ws) {
  const int lane = threadIdx.x & 63;
  ws.cut.k[lane] = k;  // lanes from n on hold key 0 and never precede an entry
  wave_sync();
  int rank = 0;
  for (int j0 = 0; j0 < n; j0 += 4) {  // entries past n hold key 0 and never count
    const uint4 q = *reinterpret_cast<const uint4*>(&ws.cut.k[j0]);
    const uint32_t kq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) rank += (kq[i] > k || (kq[i] == k && j0 + i < lane)) ? 1 : 0;
  }
  if (lane < n) {
    ws.cut.ks[rank] = k;
    ws.cut.ws[rank] = wt;
  }
  wave_sync();
  const uint32_t ks = lane < n ? ws.cut.ks[lane] : 0u;
  const unsigned long long inc = wave_scan_u64(lane < n ? ws.cut.ws[lane] : 0ull);
  const unsigned long long hit = __ballot(ks != 0u && inc >= target);
  wave_sync();
  return hit ? (uint32_t)__builtin_amdgcn_readlane((int)ks, __ffsll(hit) - 1) : 0u;
}

// Merge of one row by one wave: max, normaliser, filter threshold, kept list
// (ascending index, into the scratch lists), the probability of the drafted
// token, and the row record.  Returns false, having written nothing, when the
// candidate lists cannot decide the threshold this way (the block-level merge
// then takes the row).
template <int DT, int MODE, class Sink>
__device__ __forceinline__ bool wave_row(const Args& a, int rl, int xtok, WaveRowSm& ws, RowRec& rr,
                                         const Sink& sink, const double* tab) {
  constexpr bool FILT = MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP;
  const int lane = threadIdx.x & 63, nch = a.nchunks;
  const ChunkRec* cr = a.chunk + (size_t)rl * nch;
  const bool hx = xtok >= 0 && xtok < a.V;
  const RowT rt = row_temp(a, rl);
  const double invT = rt.invT;
  const double A64 = invT * 92.33248261689366;  // 64 log2(e) / T: exp((x - m) / T) = exp2_64((x - m) * A64)

  // one round trip: the chunk records (chunk lane + 64 i), the drafted
  // token's logit and the speculated list entries.  Every load is a buffer
  // load ranged to what it reads (past the end it returns zeros without a
  // memory access), issued before any of their data is used: loads under
  // per-lane conditions were each waited for before the next was issued.
  constexpr bool TOPKM = MODE == M_TOPK || MODE == M_TOPKP;
  const __amdgpu_buffer_rsrc_t rrec =
      __builtin_amdgcn_make_buffer_rsrc((void*)cr, (short)0, nch * (int)sizeof(ChunkRec), 0x00020000);
  u32x4 rA[4], rB[4];  // the two 16-byte halves of record lane + 64 i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rA[i] = u32x4{0u, 0u, 0u, 0u};
    rB[i] = u32x4{0u, 0u, 0u, 0u};
    if (64 * i < nch) {  // uniform
      const int off = (lane + 64 * i) * (int)sizeof(ChunkRec);
      const auto va = __builtin_amdgcn_raw_buffer_load_b128(rrec, off, 0, 0);
      rA[i] = u32x4{va[0], va[1], va[2], va[3]};
      if (FILT || MODE == M_GREEDY) {
        const auto vb = __builtin_amdgcn_raw_buffer_load_b128(rrec, off + 16, 0, 0);
        rB[i] = u32x4{vb[0], vb[1], vb[2], vb[3]};
      }
    }
  }
  // top-k: the chunks' largest thread maxima (rows of at most CTOP_CHUNKS chunks)
  u32x4 ctq[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
  const bool use_top = TOPKM && nch <= CTOP_CHUNKS && nch * CTOP >= a.top_k;
  if (use_top) {
    const __amdgpu_buffer_rsrc_t rct = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.ctop + (size_t)rl * nch * CTOP), (short)0, nch * CTOP * 4, 0x00020000);
    const auto v0 = __builtin_amdgcn_raw_buffer_load_b128(rct, lane * CTOP * 4, 0, 0);
    const auto v1 = __builtin_amdgcn_raw_buffer_load_b128(rct, lane * CTOP * 4 + 16, 0, 0);
    ctq[0] = u32x4{v0[0], v0[1], v0[2], v0[3]};
    ctq[1] = u32x4{v1[0], v1[1], v1[2], v1[3]};
  }
  // the drafted token's logit (its index clamped into the row; unused when
  // the token is outside it)
  uint32_t lxw = 0u;
  if (MODE != M_GREEDY) {
    constexpr int ESZ = ElemT<DT>::ESZ;
    const __amdgpu_buffer_rsrc_t rrow =
        __builtin_amdgcn_make_buffer_rsrc((void*)row_ptr(a, rl, ESZ), (short)0, a.V * ESZ, 0x00020000);
    const int xc = hx ? xtok : 0;
    lxw = DT == D_BF16 ? ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rrow, xc * 2, 0, 0) << 16)
                       : __builtin_amdgcn_raw_buffer_load_b32(rrow, xc * 4, 0, 0);
  }
  // with them, speculatively, the first SE entries of the first SPECC
  // chunks' lists (most top-p lists are shorter than 32 units, top-k lists
  // than 64): one round trip for most rows.  Load i holds entry lane % SE of
  // chunk i * SPL + lane / SE.
  constexpr int SPECC = 16;
  constexpr int SE = MODE == M_TOPP ? 32 : 64, SPL = 64 / SE, NSPEC = SPECC / SPL;
  uint64_t spec[NSPEC];
  const uint64_t* cand = a.cand + (size_t)rl * nch * CAND_CAP;
  if (FILT) {
    const __amdgpu_buffer_rsrc_t rsp =
        __builtin_amdgcn_make_buffer_rsrc((void*)cand, (short)0, nch * CAND_CAP * 8, 0x00020000);
#pragma unroll
    for (int i = 0; i < NSPEC; ++i) {
      const int c = i * SPL + lane / SE;
      const auto v = __builtin_amdgcn_raw_buffer_load_b64(rsp, (c * CAND_CAP + lane % SE) * 8, 0, 0);
      spec[i] = ((uint64_t)v[1] << 32) | v[0];
    }
  }
  // the records' fields (defaults for chunks past the row's)
  float cm[4];
  double cs[4];
  uint32_t cb[4];
  int cn[4], carg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool ok = lane + 64 * i < nch;
    cm[i] = ok ? __uint_as_float(rA[i][2]) : -INFINITY;
    cs[i] = ok ? __longlong_as_double((long long)(((uint64_t)rA[i][1] << 32) | rA[i][0])) : 0.0;
    cb[i] = ok ? rA[i][3] : 0u;
    cn[i] = ok ? min((int)rB[i][0], CAND_CAP) : 0;
    carg[i] = ok ? (int)rB[i][1] : INT_MAX;
  }
  const float lx = (MODE != M_GREEDY && hx) ? __uint_as_float(lxw) : -INFINITY;

  const float m = dpp_wave_fmax(fmaxf(fmaxf(cm[0], cm[1]), fmaxf(cm[2], cm[3])));
  rr.S = 0.0;
  rr.S_kept = 0.0;
  rr.px = 0.0;
  rr.m = m;
  rr.tau = 0u;
  rr.nkept = 0;
  rr.flags = 0;
  rr.arg = 0;
  rr.pad = 0;
  bool bad = !(m > -INFINITY && m < INFINITY);
  if (MODE == M_PLAIN || MODE == M_TOPP) {
    double sl = 0.0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (64 * i < nch) sl += chunk_weight_tab(cs[i], cm[i], m, rt.c2, invT, tab);  // uniform
    const double S = dpp_wave_sum(sl);
    rr.S = S;
    if (!(S > 0.0 && S < INFINITY)) bad = true;
  }
  if (MODE == M_GREEDY) {
    int best = INT_MAX;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (cm[i] == m) best = min(best, carg[i]);
    best = wave_min(best);
    rr.arg = best == INT_MAX ? 0 : best;
  }

  if (FILT && !bad) {
    // every finite logit with key >= lo is a candidate of its chunk; a chunk
    // whose max lies below lo holds none of them
    uint32_t lo = dpp_wave_umax(max(max(cb[0], cb[1]), max(cb[2], cb[3])));
    if (MODE == M_TOPP) lo = max(lo, ord_key(m - rt.win));
    if (TOPKM && use_top) {
      // the k-th largest of the chunks' recorded maxima (logits of the row)
      // is at most the row's k-th largest logit: a tighter bound than any
      // single chunk's
      const uint32_t ck[CTOP] = {ctq[0][0], ctq[0][1], ctq[0][2], ctq[0][3], ctq[1][0], ctq[1][1], ctq[1][2], ctq[1][3]};
      unsigned long long cw1[CTOP];
#pragma unroll
      for (int i = 0; i < CTOP; ++i) cw1[i] = ck[i] > KEY_NEG_INF ? 1ull : 0ull;
      lo = max(lo, wave_radix<CTOP>(ck, cw1, (unsigned long long)a.top_k, ws.hist));
      wave_sync();
    }
    // a chunk whose max lies below lo holds none of them
    int ce4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ce4[i] = (cn[i] > 0 && ord_key(cm[i]) >= lo) ? cn[i] : 0;
    int n = 0;
    auto take = [&](uint64_t raw, bool valid) {
      const uint64_t ent = valid ? cand_entry_key(raw) : 0ull;
      const bool pr = valid && (uint32_t)(ent >> 32) >= lo;
      const unsigned long long bm = __ballot(pr);
      const int pos =
          n + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
      if (pr && pos < KEEP_CAP) ws.keys[pos] = ent;
      n += __popcll(bm);
    };
    bool more = nch > SPECC;
    // the speculated entries of the chunks that hold candidates (most chunks
    // of a row hold none: their max lies below lo); chunk c < 64 lives in lane c
#pragma unroll
    for (int i = 0; i < NSPEC; ++i) {
      const int ce0 = __builtin_amdgcn_readlane(ce4[0], i * SPL);
      const int ce1 = SPL == 2 ? __builtin_amdgcn_readlane(ce4[0], i * SPL + 1) : 0;
      if (ce0 == 0 && ce1 == 0) continue;
      more |= ce0 > SE || ce1 > SE;
      take(spec[i], (lane % SE) < (lane / SE == 0 ? ce0 : ce1));
    }
    if (more) {
      // the rest: chunks past the speculated ones, entries past the first SE
      for (int c = 0; c < nch; ++c) {
        const int cv = c < 64 ? ce4[0] : c < 128 ? ce4[1] : c < 192 ? ce4[2] : ce4[3];
        const int cec = __builtin_amdgcn_readlane(cv, c & 63);
        for (int e0 = c < SPECC ? SE : 0; e0 < cec; e0 += 64) {
          const int e = e0 + lane;
          take(e < cec ? cand[(size_t)c * CAND_CAP + e] : 0ull, e < cec);
        }
      }
    }
    wave_sync();
    if (n > KEEP_CAP) return false;
    if (a.ulen > 1) {
      // read the candidate units back: their logits at or above lo are the
      // candidates (one 16-byte load per unit, all in flight together)
      constexpr int UL = 16 / ElemT<DT>::ESZ;
      const char* rp = row_ptr(a, rl, ElemT<DT>::ESZ);
      uint4 raw[WR_EPL];
      int st[WR_EPL];
#pragma unroll
      for (int r = 0; r < WR_EPL; ++r) {
        const int e = lane + 64 * r;
        st[r] = -1;
        raw[r] = make_uint4(0u, 0u, 0u, 0u);
        if (e < n) {
          st[r] = (int)(uint32_t)ws.keys[e];
          raw[r] = *reinterpret_cast<const uint4*>(rp + (size_t)st[r] * ElemT<DT>::ESZ);
        }
      }
      wave_sync();
      int ne = 0;
#pragma unroll
      for (int r = 0; r < WR_EPL; ++r) {
        if (64 * r >= n) break;  // no units in this slot on any lane
        uint64_t xv[UL];
        bool xp[UL];
#pragma unroll
        for (int i = 0; i < UL; ++i) {
          const float x = unit_elem<DT>(raw[r], i);
          const uint32_t key = ord_key(x);
          xp[i] = st[r] >= 0 && key >= lo && x > -INFINITY;
          xv[i] = ((uint64_t)key << 32) | (uint32_t)(st[r] + i);
        }
        ne = wave_append(xv, xp, ws.keys, ne, KEEP_CAP);
      }
      if (ne > KEEP_CAP) return false;
      n = ne;
      wave_sync();
    }
    uint32_t ek[WR_EPL];
    int ei[WR_EPL];
    double ew[WR_EPL];  // exp((x - m) / T)
#pragma unroll
    for (int r = 0; r < WR_EPL; ++r) {
      const int e = lane + 64 * r;
      ek[r] = 0u;
      ei[r] = 0;
      ew[r] = 0.0;
      if (64 * r < n) {
        const uint64_t v = e < n ? ws.keys[e] : 0ull;
        ek[r] = (uint32_t)(v >> 32);
        ei[r] = (int)(uint32_t)v;
        ew[r] = e < n ? exp2_64(((double)key_val(ek[r]) - (double)m) * A64, tab) : 0.0;
      }
    }
    wave_sync();
    unsigned long long wt[WR_EPL];
    uint32_t tau = lo;
    double snorm = rr.S;  // top-p normaliser
    if (MODE == M_TOPK || MODE == M_TOPKP) {
      // k-th largest key among the candidates, ties kept
#pragma unroll
      for (int r = 0; r < WR_EPL; ++r) wt[r] = ek[r] != 0u ? 1ull : 0ull;
      const uint32_t tk = n <= 64 ? wave_cut64(ek[0], wt[0], (unsigned long long)a.top_k, n, ws)
                                  : wave_radix(ek, wt, (unsigned long long)a.top_k, ws.hist);
      if (tk == 0u) {
        // fewer than k candidates: with every bound at -inf the row has fewer
        // than k finite logits and all are kept; otherwise undecided here
        if (lo > KEY_NEG_INF) return false;
        tau = KEY_NEG_INF;
      } else {
        tau = tk;
      }
      if (MODE == M_TOPKP) {
        double sk = 0.0;
#pragma unroll
        for (int r = 0; r < WR_EPL; ++r)
          if (ek[r] != 0u && ek[r] >= tau) sk += ew[r];
        snorm = dpp_wave_sum(sk);
      }
    }
    if (MODE == M_TOPP || MODE == M_TOPKP) {
      // smallest descending prefix whose mass reaches top_p, ties included
      uint32_t ekp[WR_EPL];
#pragma unroll
      for (int r = 0; r < WR_EPL; ++r) ekp[r] = ek[r] >= tau ? ek[r] : 0u;
      uint32_t tp;
      const unsigned long long target = (unsigned long long)(a.top_p * MASS_SCALE);
      if (n <= 64) {
        const unsigned long long w0 = ekp[0] != 0u ? (unsigned long long)(ew[0] / snorm * MASS_SCALE) : 0ull;
        tp = wave_cut64(ekp[0], w0, target, n, ws);
      } else {
#pragma unroll
        for (int r = 0; r < WR_EPL; ++r)
          wt[r] = ekp[r] != 0u ? (unsigned long long)(ew[r] / snorm * MASS_SCALE) : 0ull;
        tp = n <= 128 ? wave_walk<2>(ekp, wt, target) : wave_walk<WR_EPL>(ekp, wt, target);
        if (tp == 1u) tp = wave_radix(ekp, wt, target, ws.hist);
      }
      if (tp == 0u) {
        if (MODE == M_TOPP) return false;  // the nucleus reaches below the candidate window
        // top-k then top-p: round-off kept the top-k mass just below top_p; keep the top-k set
      } else {
        tau = max(tau, tp);
      }
    }
    // kept set: candidates at or above tau
    int nk = 0;
    double skl = 0.0;
    bool kp[WR_EPL];
    wave_sync();
#pragma unroll
    for (int r = 0; r < WR_EPL; ++r) {
      kp[r] = ek[r] != 0u && ek[r] >= tau;
      if (kp[r]) skl += ew[r];
      const unsigned long long bm = __ballot(kp[r]);
      if (kp[r]) {
        const int pos =
            nk + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
        ws.kept[pos] = ei[r];
      }
      nk += __popcll(bm);
    }
    const double skept = dpp_wave_sum(skl);
    wave_sync();
    // position in ascending index order = number of kept indices below it
    int pos[WR_EPL];
#pragma unroll
    for (int r = 0; r < WR_EPL; ++r) pos[r] = 0;
#pragma unroll
    for (int r = 0; r < WR_EPL; ++r) {
      if (64 * r >= n) break;  // no entries in this slot on any lane
      for (int j0 = 0; j0 < nk; j0 += 4) {
        const int4 q = *reinterpret_cast<const int4*>(&ws.kept[j0]);
        const int kq[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) pos[r] += (j0 + i < nk && kq[i] < ei[r]) ? 1 : 0;
      }
    }
#pragma unroll
    for (int r = 0; r < WR_EPL; ++r)
      if (kp[r]) sink.put(nk, pos[r], ei[r], ew[r] / skept);
    rr.tau = tau;
    rr.S_kept = skept;
    rr.nkept = nk;
  }
  if (!bad && hx) {
    if (MODE == M_GREEDY) {
      rr.px = xtok == rr.arg ? 1.0 : 0.0;
    } else if (ord_key(lx) >= rr.tau) {
      rr.px = exp2_64(((double)lx - (double)m) * A64, tab) / (MODE == M_PLAIN ? rr.S : rr.S_kept);
    }
  }
  if (bad) rr.flags |= RF_BAD;
  if (lane == 0) store_row(&a.row[rl], rr);
  return true;
}

// Row merges without sequences (sv_filtered_probs): one workgroup per row,
// its first wave merges the row (wave_row); when the candidate lists cannot
// decide the cut the whole block merges it (row_finalize).  Only the row
// records are kept (the probabilities kernel reads them).
struct RowKSm {
  union {
    WaveRowSm w;  // wave-level merge
    Smem blk;     // block-level merge
  };
  double etab[64];  // 2^(j/64) for exp2_64
  int32_t fast;
};

template <int DT, int MODE>
__global__ void __launch_bounds__(WG) row_kernel(Args a) {
  __shared__ RowKSm sm;
  const int t = threadIdx.x;
  const int rl = (int)blockIdx.x;
  if (t < 64) {
    sm.etab[t] = exp2((double)t / 64.0);  // read by this wave only
    wave_sync();
    RowRec rr;
    const bool ok = wave_row<DT, MODE>(a, rl, -1, sm.w, rr, NoSink{}, sm.etab);
    if (t == 0) sm.fast = ok;
  }
  __syncthreads();
  if (!sm.fast) (void)row_finalize<DT, MODE, WG>(a, rl, -1, sm.blk, NoSink{});
}

// Final draw from kept lists by one wave (filtered rows): residual
// max(0, p - q) over the target's kept tokens, or p itself (bonus, or an
// empty residual); inverse CDF in ascending vocabulary order.  *Zout gets the
// total weight, *wout the drawn token's weight.
// qrow: the draft distribution as a probability row; q of each kept target
// token is then read from it (the draft list is not used).
__device__ __forceinline__ int wave_list_sample(double u, const int32_t* pidx, const double* pprob, int np, const int32_t* qidx,
                                const double* qprob, int nq, bool res, double* Zout, double* wout,
                                const float* qrow = nullptr) {
  const int lane = threadIdx.x & 63;
  // entries WR_EPL * lane + r: each lane a contiguous run
  int pi[WR_EPL];
  double pp[WR_EPL], w[WR_EPL];
#pragma unroll
  for (int r = 0; r < WR_EPL; ++r) {
    const int e = WR_EPL * lane + r;
    pi[r] = e < np ? pidx[e] : 0;
    pp[r] = e < np ? pprob[e] : 0.0;
    w[r] = pp[r];
  }
  if (res) {
    double qv[WR_EPL];
    if (qrow) {
      // q read at each kept target token (one round trip)
#pragma unroll
      for (int r = 0; r < WR_EPL; ++r) qv[r] = WR_EPL * lane + r < np ? (double)qrow[pi[r]] : 0.0;
    } else {
      // q of each target token: one pass over the draft's kept list (each
      // entry read by all lanes at once)
#pragma unroll
      for (int r = 0; r < WR_EPL; ++r) qv[r] = 0.0;
      for (int j = 0; j < nq; ++j) {
        const int qi = qidx[j];
        const double qp = qprob[j];
#pragma unroll
        for (int r = 0; r < WR_EPL; ++r) qv[r] = qi == pi[r] ? qp : qv[r];
      }
    }
#pragma unroll
    for (int r = 0; r < WR_EPL; ++r) {
      if (WR_EPL * lane + r < np) {
        const double d = pp[r] - qv[r];
        w[r] = d > 0.0 ? d : 0.0;
      }
    }
  }
  double ls = 0.0;
#pragma unroll
  for (int r = 0; r < WR_EPL; ++r) ls += w[r];
  double inc = wave_scan_f64(ls);
  double Z = lane63(inc);
  if (res && !(Z > 0.0)) {  // empty residual: draw from p
    ls = 0.0;
#pragma unroll
    for (int r = 0; r < WR_EPL; ++r) {
      w[r] = pp[r];
      ls += w[r];
    }
    inc = wave_scan_f64(ls);
    Z = lane63(inc);
  }
  const double target = u * Z;
  double C = inc - ls;
  int first = INT_MAX, lastp = -1, tf = 0, tl = 0;
  double wf = 0.0, wl = 0.0;
#pragma unroll
  for (int r = 0; r < WR_EPL; ++r) {
    const int e = WR_EPL * lane + r;
    C += w[r];
    if (e < np && w[r] > 0.0) {
      lastp = e;
      tl = pi[r];
      wl = w[r];
      if (first == INT_MAX && target < C) {
        first = e;
        tf = pi[r];
        wf = w[r];
      }
    }
  }
  const unsigned long long fm = __ballot(first != INT_MAX);
  int tok;
  double wt = 0.0;
  if (fm) {
    tok = lane_bcast(tf, __ffsll(fm) - 1);
    wt = lane_bcast(wf, __ffsll(fm) - 1);
  } else {
    const unsigned long long lm = __ballot(lastp >= 0);
    tok = lm ? lane_bcast(tl, 63 - __clzll(lm)) : 0;
    wt = lm ? lane_bcast(wl, 63 - __clzll(lm)) : 0.0;
  }
  *Zout = Z;
  *wout = wt;
  return tok;
}

// Sequence b as a sentinel (n = -1, tokens -1), by the threads of one
// workgroup; its uniform-indexed outputs only (out_p and out_q are left).
__device__ void sentinel_seq(const Args& a, int b, int t) {
  const double nanv = __longlong_as_double(0x7FF8000000000000ll);
  for (int j = t; j <= a.Kmax; j += blockDim.x) a.out_tok[(size_t)b * (a.Kmax + 1) + j] = -1;
  if (t == 0) {
    if (a.out_n) a.out_n[b] = -1;
    if (a.out_z) a.out_z[b] = nanv;
    if (a.out_px) a.out_px[b] = nanv;
    SeqRec sr = {};
    sr.n = -1;
    sr.flags = RF_BAD;
    a.seq[b] = sr;
  }
}

// ---------------------------------------------------------------------------
// sequence kernel: one workgroup per sequence merges all of the sequence's
// rows at once (one wave per row) and then runs its accept tests, its
// first-rejection scan and its draw, with everything in the workgroup's LDS
// ---------------------------------------------------------------------------
constexpr int SQ_WAVES = 16;              // waves of a sequence workgroup (rows merged at once)
constexpr int SQ_BS = SQ_WAVES * 64;      // its threads
constexpr int SQ_WAVES_SMALL = 8;         // waves of the workgroups of sequences of at most 8 rows
constexpr int SQ_SLOTS = SQ_WAVES;        // rows whose kept lists can stay in LDS
constexpr int SQ_SLOT_CAP = 64;           // ... when they have at most this many entries
static_assert(SQ_BS <= 1024, "Smem.scan holds one entry per thread");

struct SeqKSm {
  union {
    WaveRowSm w[SQ_WAVES];  // the waves' row merges
    Smem blk;               // block-level merge, list copies and full-row draw
  };
  int32_t kidx[SQ_SLOTS][SQ_SLOT_CAP];
  double kprob[SQ_SLOTS][SQ_SLOT_CAP];
  // per row of the sequence: target rows 0..K, then draft rows K+1..2K (with
  // q given as probabilities, slot K+1+i holds the given q(x_i))
  double px[MAX_RPS];   // p or q of the row's drafted token
  double rs[MAX_RPS];   // full-row normaliser (unfiltered rows: for the draw)
  float rm[MAX_RPS];    // row maximum
  int32_t rf[MAX_RPS];  // row flags
  int32_t nk[MAX_RPS];  // kept-list length (-1: too large for a list)
  int32_t arg[MAX_RPS]; // greedy arg-max
  int32_t x[MAX_K];
  float u[MAX_K + 1];
  double etab[64];  // 2^(j/64) for exp2_64
  uint32_t fail[(MAX_RPS + 31) / 32];  // rows the waves could not merge from the candidate lists
  int32_t n, big;
};

// The kept list of the sequence's row j: in the workgroup's LDS slot j when
// j < SQ_SLOTS and the list has at most SQ_SLOT_CAP entries, otherwise in the
// row's scratch list (read back by the same workgroup only).
struct SeqSink {
  SeqKSm& sm;
  int j;
  int32_t* gidx;
  double* gprob;
  __device__ __forceinline__ void put(int nk, int pos, int32_t idx, double prob) const {
    if (j < SQ_SLOTS && nk <= SQ_SLOT_CAP) {
      sm.kidx[j][pos] = idx;
      sm.kprob[j][pos] = prob;
    } else {
      gidx[pos] = idx;
      gprob[pos] = prob;
    }
  }
};
__device__ __forceinline__ SeqSink seq_sink(const Args& a, SeqKSm& sm, int j, int rl) {
  return SeqSink{sm, j, a.kidx + (size_t)rl * KEEP_CAP, a.kprob + (size_t)rl * KEEP_CAP};
}

// One workgroup of NW waves per sequence.  Each wave merges one of the
// sequence's rows, and one more with NR = 2 (wave_row: the chunk records and most
// candidate units in one round trip, the units' logits in a second); a row
// the lists cannot decide is merged afterwards by the whole workgroup
// (row_finalize).  Then the first wave runs the accept tests, the
// first-rejection scan and the draw from the kept lists (from full rows,
// by the whole workgroup, when a kept set is too large for a list;
// unfiltered rows: the sampling kernel draws afterwards).  No data passes
// between workgroups.
// LAY (BatchLayout): rectangular, ragged (offsets validated by the streaming
// kernel's first workgroup), or rectangular with q given as probabilities
// (no draft rows: each target row i < K reads the given q(x_i), and the
// residual draw reads q at the target's kept tokens).
// NR: rows per wave (2 for sequences of more than SQ_WAVES rows; a separate
// instantiation, so that the common case keeps its register allocation).
// NW: waves of the workgroup, SQ_WAVES, or SQ_WAVES_SMALL when every
// sequence of the call has at most that many rows: at 128 registers a lane
// one workgroup of 16 waves fills a compute unit's register file, and two
// of 8 waves share it (the drafting draw's one-row sequences, or K <= 3,
// then take one round of workgroups instead of two).
template <int DT, int MODE, int LAY, int NR, int NW>
__global__ void __launch_bounds__(NW * 64, 4) seq_kernel(Args a) {
  constexpr int BS = NW * 64;
  __shared__ SeqKSm sm;
  constexpr int ESZ = ElemT<DT>::ESZ;
  constexpr bool FILT = MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP;
  constexpr bool RAG = LAY == LAY_RAG, QP = LAY == LAY_QP;
  // the wave index, made a scalar (the compiler does not see that t >> 6 is
  // the same in every lane of a wave): the per-row code then branches and
  // indexes on scalars
  const int t = threadIdx.x, w = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int b = (int)blockIdx.x;
  if (RAG && a.cflag[0] == 0) {
    // offsets that describe no packing: every sequence is a sentinel
    sentinel_seq(a, b, t);
    return;
  }
  const SeqGeo g = seq_geo<RAG>(a, b);
  const int K = g.K;
  const int rps = (MODE == M_GREEDY || QP) ? K + 1 : 2 * K + 1;
  // rows j >= NR NW (sequences of more rows than the waves take) are
  // merged by the whole workgroup below, one after another
  if (t < (MAX_RPS + 31) / 32) {
    const int j0 = 32 * t, nw = NR * NW;
    sm.fail[t] = j0 >= nw ? ~0u : (nw - j0 >= 32 ? 0u : ~0u << (nw - j0));
  }
  if (t < K) sm.x[t] = a.X[(size_t)g.x0 + t];
  if (t >= 256 && t - 256 <= K) sm.u[t - 256] = a.U[(size_t)g.t0 + (t - 256)];
  if (t >= BS - 64) sm.etab[t - (BS - 64)] = exp2((double)(t - (BS - 64)) / 64.0);
  __syncthreads();

  // ---- the sequence's rows, one wave each: wave w merges row w, and (NR = 2)
  // row w + NW when the sequence has that many
  auto merge_row = [&](const int j) {
    const int rl = seq_row<RAG>(a, g, j);
    const int i = j <= K ? j : j - K - 1;  // position of the row
    const int xtok = i < K ? sm.x[i] : -1;
    RowRec rr;
    const bool ok = wave_row<DT, MODE>(a, rl, xtok, sm.w[w], rr, seq_sink(a, sm, j, rl), sm.etab);
    // a kept list written to the scratch (too long for an LDS slot) is read
    // back by this workgroup below: the wave that wrote it waits for its
    // stores (no other wave's stores need waiting for)
    if (FILT && ok && (j >= SQ_SLOTS || rr.nkept > SQ_SLOT_CAP)) __builtin_amdgcn_s_waitcnt(0);
    if (lane == 0) {
      if (ok) {
        sm.px[j] = rr.px;
        sm.rf[j] = rr.flags;
        sm.nk[j] = rr.nkept;
        sm.arg[j] = rr.arg;
        sm.rm[j] = rr.m;
        sm.rs[j] = rr.S;
      } else {
        atomicOr(&sm.fail[j >> 5], 1u << (j & 31));
      }
      // q(x_i) from the given draft row
      if (QP && i < K && j <= K)
        sm.px[K + 1 + i] = (xtok >= 0 && xtok < a.V) ? (double)a.qprob[(size_t)(g.x0 + i) * a.V + xtok] : 0.0;
    }
  };
  // Wave w runs on SIMD w % 4.  With 4k + 1 rows (2K + 1 at even K) SIMD 0
  // runs one row wave more than the others: it takes the first rows (target
  // rows, whose merges are lighter than the draft rows'), and the other
  // SIMDs take the rest slot by slot, a target row and draft rows each.
  const bool spread = NR == 1 && (rps & 3) == 1;
  const int wrow = !spread ? w : (w & 3) == 0 ? (w >> 2) : (rps + 3) / 4 + 3 * (w >> 2) + (w & 3) - 1;
  if (w < rps) merge_row(wrow);
  if (NR > 1 && w + NW < rps) merge_row(w + NW);
  __syncthreads();
  // ---- rows the candidate lists could not decide: the whole workgroup
  for (int wd = 0; 32 * wd < rps; ++wd) {
    uint32_t bits = sm.fail[wd];  // the same in every thread
    if (rps - 32 * wd < 32) bits &= (1u << (rps - 32 * wd)) - 1u;
    // (rare: marked unlikely, so that the register spills this block-level
    // path needs are placed on it and not on the common path)
    while (__builtin_expect(bits != 0u, 0)) {
      const int j = 32 * wd + __ffs(bits) - 1;
      bits &= bits - 1u;
      const int rl = seq_row<RAG>(a, g, j);
      const int i = j <= K ? j : j - K - 1;
      const int xtok = i < K ? sm.x[i] : -1;
      const RowRec rr = row_finalize<DT, MODE, BS>(a, rl, xtok, sm.blk, seq_sink(a, sm, j, rl));
      if (t == 0) {
        sm.px[j] = rr.px;
        sm.rf[j] = rr.flags;
        sm.nk[j] = rr.nkept;
        sm.arg[j] = rr.arg;
        sm.rm[j] = rr.m;
        sm.rs[j] = rr.S;
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- the sequence
  if (w == 0) {
    // accept tests: draft i is accepted iff u_i * q_i(x_i) < p_i(x_i)
    bool rej = false, badx = false;
    if (lane < K) {
      const double p = sm.px[lane];
      rej = MODE == M_GREEDY ? !(p > 0.0) : !((double)sm.u[lane] * sm.px[K + 1 + lane] < p);
      badx = sm.x[lane] < 0 || sm.x[lane] >= a.V;
    }
    bool badr = false;
    for (int j = lane; j < rps; j += 64) badr |= (sm.rf[j] & RF_BAD) != 0;
    const unsigned long long rm = __ballot(rej);
    const bool bad = __ballot(badx || badr) != 0ull;
    const int n = bad ? -1 : (rm ? __ffsll(rm) - 1 : K);
    int32_t* ot = a.out_tok + (size_t)b * (a.Kmax + 1);
    const double nanv = __longlong_as_double(0x7FF8000000000000ll);
    if (lane < K) {
      if (a.out_p) a.out_p[(size_t)g.x0 + lane] = n < 0 ? nanv : sm.px[lane];
      if (a.out_q) a.out_q[(size_t)g.x0 + lane] = (n < 0 || MODE == M_GREEDY) ? nanv : sm.px[K + 1 + lane];
    }
    for (int j = lane; j <= a.Kmax; j += 64) {
      if (n < 0 || j > n) ot[j] = -1;
      else if (j < n) ot[j] = sm.x[j];
    }
    int big = 0;
    if (lane == 0) {
      if (a.out_n) a.out_n[b] = n;
      SeqRec sr = {};
      sr.n = n;
      sr.flags = n < 0 ? RF_BAD : 0;
      if (MODE == M_PLAIN && n >= 0) {
        // the unfiltered draw's rows: p at position n; q the draft row n
        // (or its given probability row) after a rejection
        const bool res = n < K;
        sr.rp = seq_row<RAG>(a, g, n);
        sr.mp = sm.rm[n];
        sr.sp = sm.rs[n];
        sr.rq = QP ? g.x0 + (res ? n : 0) : res ? seq_row<RAG>(a, g, K + 1 + n) : sr.rp;
        sr.mq = (!QP && res) ? sm.rm[K + 1 + n] : 0.0f;
        sr.sq = (!QP && res) ? sm.rs[K + 1 + n] : 1.0;
        sr.tu = g.t0 + K;
        sr.k = K;
      }
      a.seq[b] = sr;
      if (n < 0 && a.out_z) a.out_z[b] = nanv;
      if (n < 0 && a.out_px) a.out_px[b] = nanv;
      if (n >= 0 && MODE == M_GREEDY) {
        ot[n] = sm.arg[n];
        if (a.out_z) a.out_z[b] = 1.0;
        if (a.out_px) a.out_px[b] = 1.0;
      }
    }
    if (FILT && n >= 0) {
      const bool res = n < K;
      const int jq = res ? K + 1 + n : n;
      const int np = sm.nk[n], nq = QP ? 0 : sm.nk[jq];
      if (np < 0 || (res && nq < 0)) {
        big = 1;
      } else {
        // each list from its LDS slot, or copied from the scratch (one round trip)
        SmemSeq& q = sm.blk.q;
        const int32_t* pidx = sm.kidx[n < SQ_SLOTS ? n : 0];
        const double* pprob = sm.kprob[n < SQ_SLOTS ? n : 0];
        const int32_t* qidx = sm.kidx[jq < SQ_SLOTS ? jq : 0];
        const double* qprob = sm.kprob[jq < SQ_SLOTS ? jq : 0];
        const bool pg = !(n < SQ_SLOTS && np <= SQ_SLOT_CAP);
        const bool qg = res && !QP && !(jq < SQ_SLOTS && nq <= SQ_SLOT_CAP);
        if (pg) {
          const size_t op = (size_t)seq_row<RAG>(a, g, n) * KEEP_CAP;
          for (int e = lane; e < np; e += 64) {
            q.pidx[e] = ld_dev(&a.kidx[op + e]);
            q.pprob[e] = ld_dev(&a.kprob[op + e]);
          }
          pidx = q.pidx;
          pprob = q.pprob;
        }
        if (qg) {
          const size_t oq = (size_t)seq_row<RAG>(a, g, jq) * KEEP_CAP;
          for (int e = lane; e < nq; e += 64) {
            q.qidx[e] = ld_dev(&a.kidx[oq + e]);
            q.qprob[e] = ld_dev(&a.kprob[oq + e]);
          }
          qidx = q.qidx;
          qprob = q.qprob;
        }
        if (QP) {
          qidx = pidx;
          qprob = pprob;
        }
        wave_sync();
        double Z, wtok;
        const float* qrow = QP ? a.qprob + (size_t)(g.x0 + n) * a.V : nullptr;
        const int tok = wave_list_sample((double)sm.u[K], pidx, pprob, np, qidx, qprob, nq, res, &Z, &wtok, qrow);
        if (lane == 0) {
          ot[n] = tok;
          if (a.out_z) a.out_z[b] = Z;
          if (a.out_px) a.out_px[b] = res ? nanv : wtok;  // a bonus draw's weight is the kept probability
        }
      }
    }
    if (lane == 0) {
      sm.big = big;
      sm.n = n;
    }
  }
  __syncthreads();
  if (__builtin_expect(FILT && sm.big, 0)) {
    // a kept set too large for a list: the whole workgroup draws from the full rows
    const int n = sm.n;
    const bool res = n < K;
    const int jq = res ? K + 1 + n : n;
    const int rn = seq_row<RAG>(a, g, n), rq = QP ? rn : seq_row<RAG>(a, g, jq);
    set_draw_row(&a.row[rn], true, 0, row_temp(a, rn).invT, sm.blk);
    if (QP) set_draw_prob_row(a.qprob + (size_t)(g.x0 + (res ? n : 0)) * a.V, 1, sm.blk);
    else set_draw_row(&a.row[rq], true, 1, row_temp(a, rq).invT, sm.blk);
    double Z;
    const int tok = full_row_sample<DT, BS>(a, (double)sm.u[K], row_ptr(a, rn, ESZ), row_ptr(a, rq, ESZ), res,
                                               sm.blk, &Z);
    if (t == 0) {
      a.out_tok[(size_t)b * (a.Kmax + 1) + n] = tok;
      if (a.out_z) a.out_z[b] = Z;
      if (a.out_px)
        a.out_px[b] = res ? __longlong_as_double(0x7FF8000000000000ll)
                          : kept_prob<DT>(row_ptr(a, rn, ESZ), tok, load_row(&a.row[rn]), true, row_temp(a, rn).invT);
    }
  }
}

// Weights of the unfiltered draw: p_j = exp((x_j - m) / T) / S from the
// row's record, and for a residual max(0, p_j - q_j) with q_j likewise (or
// read from a row of probabilities, QP).  exp_tab and the reciprocals of the
// normalisers keep this pass, which touches every logit of two rows, light.
// p_j = exp((x_j - m) / T) / S = 2^(y / 64) with y = x_j * A + B, where
// A = 64 log2(e) / T and B = -m A - 64 log2(S): one fma and exp2_64 per
// weight.  (The rounding of A, B and y leaves a relative error of a few
// 1e-15 in each weight.)
struct PlainW {
  double ap, bp;  // p's row
  double aq, bq;  // q's row (logits)
};
__device__ __forceinline__ void plain_affine(float m, double invT, double S, double& A, double& B) {
  A = invT * 92.33248261689366;  // 64 log2(e)
  B = fma(-(double)m, A, -64.0 * log2(S));
}
template <bool QP>
__device__ __forceinline__ double plain_w(float xp, float xq, const PlainW& c, bool res, const double* tab) {
  const double p = exp2_64(fma((double)xp, c.ap, c.bp), tab);
  if (!res) return p;
  const double q = QP ? (double)xq : exp2_64(fma((double)xq, c.aq, c.bq), tab);
  const double d = p - q;
  return d > 0.0 ? d : 0.0;
}
template <int DT, bool QP>
__device__ __forceinline__ double plain_weight(const char* pr, const char* qr, int j, const PlainW& c, bool res,
                                               const double* tab) {
  const float xp = load_elem<DT>(pr, j);
  const float xq = !res ? 0.0f : QP ? reinterpret_cast<const float*>(qr)[j] : load_elem<DT>(qr, j);
  return plain_w<QP>(xp, xq, c, res, tab);
}
template <int DT, int LAY>
__global__ void __launch_bounds__(WG) sample_kernel(Args a) {
  constexpr bool QP = LAY == LAY_QP;
  __shared__ Smem sm;
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x;
  const int b = (int)(blockIdx.x / (unsigned)a.nsw);
  const int cb = ((int)blockIdx.x - b * a.nsw) * a.spw;  // first sampling chunk of this workgroup
  const int nseg = a.nsc * SEG_PER_SCE;
  const SeqRec sr = a.seq[b];  // written by the row merge: rows, normalisers, uniform
  const int n = sr.n;
  const bool active = n >= 0;
  const bool res = active && n < sr.k;
  build_exp_tab(sm.etab);
  PlainW cw = {0.0, 0.0, 0.0, 0.0};
  if (active) plain_affine(sr.mp, row_temp(a, sr.rp).invT, sr.sp, cw.ap, cw.bp);
  if (active && res && !QP) plain_affine(sr.mq, row_temp(a, sr.rq).invT, sr.sq, cw.aq, cw.bq);
  const char* pr = active ? row_ptr(a, sr.rp, ESZ) : nullptr;
  const char* qr = !active ? nullptr
                   : QP    ? reinterpret_cast<const char*>(a.qprob + (size_t)sr.rq * a.V)
                           : row_ptr(a, sr.rq, ESZ);
  if (active) {
    // the workgroup's spw chunks of 2048 logits: every load first, then the
    // weights and one segment sum per wave and chunk
    float xp[SPW][8], xq[SPW][8];
    if (a.ulen > 1 && !QP) {
      // every load issued before any is unpacked
      Raw8<DT> rpv[SPW], rqv[SPW];
#pragma unroll
      for (int ci = 0; ci < SPW; ++ci) {
        const int j0 = (cb + ci) * SCE + t * 8;
        rpv[ci] = load8_raw<DT>(pr, ci < a.spw ? j0 : a.V, a.V);
        if (res) rqv[ci] = load8_raw<DT>(qr, ci < a.spw ? j0 : a.V, a.V);
      }
#pragma unroll
      for (int ci = 0; ci < SPW; ++ci) {
        const int j0 = (cb + ci) * SCE + t * 8;
        unpack8<DT>(rpv[ci], j0, a.V, xp[ci]);
        if (res) {
          unpack8<DT>(rqv[ci], j0, a.V, xq[ci]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xq[ci][e] = 0.0f;
        }
      }
    } else
#pragma unroll
    for (int ci = 0; ci < SPW; ++ci) {
      if (ci >= a.spw) break;  // uniform
      const int j0 = (cb + ci) * SCE + t * 8;
      load8<DT>(pr, j0, a.V, a.ulen > 1, xp[ci]);
      if (res) {
        if (QP) {
#pragma unroll
          for (int e = 0; e < 8; ++e) xq[ci][e] = j0 + e < a.V ? reinterpret_cast<const float*>(qr)[j0 + e] : 0.0f;
        } else {
          load8<DT>(qr, j0, a.V, a.ulen > 1, xq[ci]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xq[ci][e] = 0.0f;
      }
    }
#pragma unroll
    for (int ci = 0; ci < SPW; ++ci) {
      const int c = cb + ci;
      if (ci >= a.spw || c >= a.nsc) break;  // uniform
      const int j0 = c * SCE + t * 8;
      double ts = 0.0;
      int lastp = -1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double w = j0 + e < a.V ? plain_w<QP>(xp[ci][e], xq[ci][e], cw, res, sm.etab) : 0.0;
        ts += w;
        if (w > 0.0) lastp = j0 + e;
      }
      const double ss = wave_sum(ts);
      const int sl = wave_max(lastp);
      if ((t & 63) == 0) {
        const size_t sg = (size_t)b * nseg + c * SEG_PER_SCE + (t >> 6);
        st_dev(&a.seg_sum[sg], ss);
        st_dev(&a.seg_last[sg], sl);
      }
    }
  }
  if (!last_arrival(&a.smp_cnt[b], (uint32_t)a.nsw, &sm.flag)) return;
  if (!active) return;

  // The last workgroup of the sequence draws.  Wave 0 alone: no block-wide
  // scans.  Lane l sums the segments of its contiguous run, one exclusive
  // scan over the lanes gives every run's start, and the run holding u*Z
  // is walked segment by segment; the segment is then rescanned, 8 logits a
  // lane.
  const double* ssum = a.seg_sum + (size_t)b * nseg;
  const int32_t* slast = a.seg_last + (size_t)b * nseg;
  const double u = (double)a.U[sr.tu];
  const int lane = t & 63;
  int tok = 0;
  double Z = 0.0;
  if (t < 64) {
    const int per = (nseg + 63) / 64;
    const int s0 = min(lane * per, nseg), s1 = min(s0 + per, nseg);
    // the run's sums RUNQ at a time, every load of a group in flight together
    // (addresses clamped to the run; values past it are not used); the first
    // group is kept for the walk below (the whole run when per <= RUNQ)
    constexpr int RUNQ = 4;
    double loc = 0.0, rv[RUNQ];
    int lastseg = -1;
#pragma unroll
    for (int q = 0; q < RUNQ; ++q) rv[q] = 0.0;
    for (int g0 = s0; g0 < s1; g0 += RUNQ) {
      double v[RUNQ];
      int l[RUNQ];
#pragma unroll
      for (int q = 0; q < RUNQ; ++q) {
        const int sg = min(g0 + q, s1 - 1);
        v[q] = ld_dev(&ssum[sg]);
        l[q] = ld_dev(&slast[sg]);
      }
#pragma unroll
      for (int q = 0; q < RUNQ; ++q) {
        if (g0 == s0) rv[q] = v[q];
        if (g0 + q < s1) {
          loc += v[q];
          if (l[q] >= 0) lastseg = g0 + q;
        }
      }
    }
    const double incl = wave_scan_f64(loc);
    Z = lane63(incl);
    lastseg = wave_max(lastseg);
    if (lane == 0) {
      sm.d0 = Z;
      sm.i0 = lastseg;
    }
    if (Z > 0.0) {
      const double target = u * Z;
      // the run (lane) holding the target: the lanes' [previous lane's
      // inclusive sum, own inclusive sum) ranges tile [0, Z) exactly; then
      // the segment within the run (its last one if round-off in the run's
      // own sum leaves the target past it)
      const double excl = lane_bcast(incl, lane > 0 ? lane - 1 : 0);
      double run = lane > 0 ? excl : 0.0;
      int found = INT_MAX;
      double cstart = 0.0;
      if (run <= target && target < incl && s0 < s1) {
        for (int g0 = s0; g0 < s1 && found == INT_MAX; g0 += RUNQ) {
          double v[RUNQ];
#pragma unroll
          for (int q = 0; q < RUNQ; ++q) v[q] = g0 == s0 ? rv[q] : ld_dev(&ssum[min(g0 + q, s1 - 1)]);
#pragma unroll
          for (int q = 0; q < RUNQ; ++q) {
            const int sg = g0 + q;
            if (found == INT_MAX && sg < s1) {
              const double ce = run + v[q];
              if (target < ce || sg == s1 - 1) {
                found = sg;
                cstart = run;
              } else {
                run = ce;
              }
            }
          }
        }
      }
      const unsigned long long fm = __ballot(found != INT_MAX);
      if (!fm) {
        // round-off left the target past the last sum: the last positive token
        tok = lastseg >= 0 ? ld_dev(&slast[lastseg]) : 0;
      } else {
        const int src = __ffsll(fm) - 1;
        const int sf = lane_bcast(found, src);
        const double cs = lane_bcast(cstart, src);
        // rescan segment sf: logits sf*SEG + 8 lane .. + 7
        const int j0 = sf * SEG + 8 * lane;
        float xp[8], xq[8];
        load8<DT>(pr, j0, a.V, a.ulen > 1, xp);
        if (res && !QP) {
          load8<DT>(qr, j0, a.V, a.ulen > 1, xq);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            xq[e] = (res && j0 + e < a.V) ? reinterpret_cast<const float*>(qr)[j0 + e] : 0.0f;
        }
        double w8[8], ls = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          w8[e] = j0 + e < a.V ? plain_w<QP>(xp[e], xq[e], cw, res, sm.etab) : 0.0;
          ls += w8[e];
        }
        double C = cs + wave_scan_f64(ls) - ls;
        int first = INT_MAX;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          C += w8[e];
          if (first == INT_MAX && w8[e] > 0.0 && target < C) first = j0 + e;
        }
        first = wave_min(first);
        tok = first != INT_MAX ? first : ld_dev(&slast[sf]);
        if (tok < 0) tok = lastseg >= 0 ? ld_dev(&slast[lastseg]) : 0;
      }
    }
  }
  __syncthreads();
  if (!(sm.d0 > 0.0)) {
    // empty residual (round-off only): the whole workgroup draws from p
    set_draw_row(&a.row[sr.rp], false, 0, row_temp(a, sr.rp).invT, sm);
    tok = full_row_sample<DT, WG>(a, u, pr, qr, false, sm, &Z);
  }
  if (t == 0) {
    a.out_tok[(size_t)b * (a.Kmax + 1) + n] = tok;
    if (a.out_z) a.out_z[b] = Z;
    if (a.out_px)
      a.out_px[b] = res ? __longlong_as_double(0x7FF8000000000000ll) : plain_weight<DT, QP>(pr, qr, tok, cw, false, sm.etab);
  }
}

template <int DT, int MODE>
__global__ void __launch_bounds__(WG) probs_kernel(Args a) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x;
  const int rl = (int)(blockIdx.x / (unsigned)a.nsc);
  const int c = (int)blockIdx.x - rl * a.nsc;
  const RowRec R = a.row[rl];
  const char* rp = row_ptr(a, rl, ESZ);
  const bool filtered = MODE != M_PLAIN;
  for (int e = 0; e < 8; ++e) {
    const int j = c * SCE + e * WG + t;
    if (j < a.V) {
      float out;
      if (R.flags & RF_BAD) out = __int_as_float(0x7FC00000);
      else out = (float)kept_prob<DT>(rp, j, R, filtered, row_temp(a, rl).invT);
      a.out_probs[(size_t)rl * a.V + j] = out;
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
typedef void (*KFn)(Args);

template <int DT, int MODE>
static KFn pick_stream(bool vec) {
  return vec ? (KFn)stream_kernel_vec<DT, MODE> : (KFn)stream_kernel_elem<DT, MODE>;
}

template <int DT>
static KFn pick_stream_mode(int mode, bool vec) {
  switch (mode) {
    case M_PLAIN: return pick_stream<DT, M_PLAIN>(vec);
    case M_TOPK: return pick_stream<DT, M_TOPK>(vec);
    case M_TOPP: return pick_stream<DT, M_TOPP>(vec);
    case M_TOPKP: return pick_stream<DT, M_TOPKP>(vec);
    default: return pick_stream<DT, M_GREEDY>(vec);
  }
}

template <int DT, int LAY, int NR, int NW>
static KFn pick_seq(int mode) {
  switch (mode) {
    case M_PLAIN: return (KFn)seq_kernel<DT, M_PLAIN, LAY, NR, NW>;
    case M_TOPK: return (KFn)seq_kernel<DT, M_TOPK, LAY, NR, NW>;
    case M_TOPP: return (KFn)seq_kernel<DT, M_TOPP, LAY, NR, NW>;
    case M_TOPKP: return (KFn)seq_kernel<DT, M_TOPKP, LAY, NR, NW>;
    default: return (KFn)seq_kernel<DT, M_GREEDY, LAY, NR, NW>;
  }
}

template <int DT, int NR, int NW>
static KFn pick_seq_lay(int mode, int lay) {
  return lay == LAY_RAG ? pick_seq<DT, LAY_RAG, NR, NW>(mode)
         : lay == LAY_QP ? pick_seq<DT, LAY_QP, NR, NW>(mode)
                         : pick_seq<DT, LAY_RECT, NR, NW>(mode);
}

static int layout_of(const Args& a) { return a.cu ? LAY_RAG : a.qprob ? LAY_QP : LAY_RECT; }

template <int DT>
static KFn pick_row(int mode) {
  switch (mode) {
    case M_PLAIN: return (KFn)row_kernel<DT, M_PLAIN>;
    case M_TOPK: return (KFn)row_kernel<DT, M_TOPK>;
    case M_TOPP: return (KFn)row_kernel<DT, M_TOPP>;
    default: return (KFn)row_kernel<DT, M_TOPKP>;
  }
}

template <int DT>
static KFn pick_probs(int mode) {
  switch (mode) {
    case M_PLAIN: return (KFn)probs_kernel<DT, M_PLAIN>;
    case M_TOPK: return (KFn)probs_kernel<DT, M_TOPK>;
    case M_TOPP: return (KFn)probs_kernel<DT, M_TOPP>;
    default: return (KFn)probs_kernel<DT, M_TOPKP>;
  }
}

// grid: ceil(rows / NXCD) * NXCD * nchunks workgroups for a.nitems
// streaming items (stream_item).
// With events, the launch itself records the kernel's start and end in them.
hipError_t launch_stream(const Args& a, int dtype, int mode, bool vec, unsigned grid, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1) {
  KFn f = dtype == D_BF16 ? pick_stream_mode<D_BF16>(mode, vec) : pick_stream_mode<D_F32>(mode, vec);
  if (e0 || e1) {
    void* args[] = {const_cast<Args*>(&a)};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(f), dim3(grid), dim3(WG), args, 0, s, e0, e1, 0);
  }
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

// Chunk records from tile statistics: the streaming kernel's grid.
hipError_t launch_tile_chunk(const Args& a, int mode, unsigned grid, const void* R, int32_t rstride, int32_t ntg,
                             hipStream_t s) {
  const uint2* r = static_cast<const uint2*>(R);
  switch (mode) {
    case M_PLAIN: hipLaunchKernelGGL(tile_chunk_kernel<M_PLAIN>, dim3(grid), dim3(WG), 0, s, a, r, rstride, ntg); break;
    case M_TOPK: hipLaunchKernelGGL(tile_chunk_kernel<M_TOPK>, dim3(grid), dim3(WG), 0, s, a, r, rstride, ntg); break;
    case M_TOPP: hipLaunchKernelGGL(tile_chunk_kernel<M_TOPP>, dim3(grid), dim3(WG), 0, s, a, r, rstride, ntg); break;
    case M_TOPKP: hipLaunchKernelGGL(tile_chunk_kernel<M_TOPKP>, dim3(grid), dim3(WG), 0, s, a, r, rstride, ntg); break;
    default: hipLaunchKernelGGL(tile_chunk_kernel<M_GREEDY>, dim3(grid), dim3(WG), 0, s, a, r, rstride, ntg); break;
  }
  return hipGetLastError();
}

// Row merges without sequences (sv_filtered_probs): one workgroup per row.
hipError_t launch_row(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s) {
  KFn f = dtype == D_BF16 ? pick_row<D_BF16>(mode) : pick_row<D_F32>(mode);
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

// The sequences: one workgroup per sequence, of SQ_WAVES waves (two rows a
// wave for sequences of more rows than that), or of SQ_WAVES_SMALL waves
// when no sequence of the call has more rows.
hipError_t launch_seq(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s) {
  const int lay = layout_of(a);
  // the most rows a sequence of this call has
  const int rps_max = (mode == M_GREEDY || lay == LAY_QP) ? a.Kmax + 1 : 2 * a.Kmax + 1;
  KFn f;
  int nw = SQ_WAVES;
  if (rps_max > SQ_WAVES) {
    f = dtype == D_BF16 ? pick_seq_lay<D_BF16, 2, SQ_WAVES>(mode, lay) : pick_seq_lay<D_F32, 2, SQ_WAVES>(mode, lay);
  } else if (rps_max > SQ_WAVES_SMALL) {
    f = dtype == D_BF16 ? pick_seq_lay<D_BF16, 1, SQ_WAVES>(mode, lay) : pick_seq_lay<D_F32, 1, SQ_WAVES>(mode, lay);
  } else {
    f = dtype == D_BF16 ? pick_seq_lay<D_BF16, 1, SQ_WAVES_SMALL>(mode, lay)
                        : pick_seq_lay<D_F32, 1, SQ_WAVES_SMALL>(mode, lay);
    nw = SQ_WAVES_SMALL;
  }
  hipLaunchKernelGGL(f, dim3(grid), dim3(nw * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sample(const Args& a, int dtype, unsigned grid, hipStream_t s) {
  const int lay = layout_of(a);
  KFn f = dtype == D_BF16 ? (lay == LAY_RAG  ? (KFn)sample_kernel<D_BF16, LAY_RAG>
                             : lay == LAY_QP ? (KFn)sample_kernel<D_BF16, LAY_QP>
                                             : (KFn)sample_kernel<D_BF16, LAY_RECT>)
                          : (lay == LAY_RAG  ? (KFn)sample_kernel<D_F32, LAY_RAG>
                             : lay == LAY_QP ? (KFn)sample_kernel<D_F32, LAY_QP>
                                             : (KFn)sample_kernel<D_F32, LAY_RECT>);
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

// Plain read of nbytes from p, 16 KiB per workgroup with the streaming
// kernel's loads (four 16-byte non-temporal buffer loads per thread, each range ending
// with the workgroup's block, so a tail block reads zeros past the end
// without a memory access), and nothing else: the floor that the streaming
// pass's loads alone reach.  The xor of a block's words is written to
// out[block] only when it equals key, so that the loads cannot be dropped and
// almost nothing is written.
__global__ void __launch_bounds__(WG) read_kernel(const char* p, int64_t nbytes, uint32_t key, uint32_t* out) {
  const int64_t b0 = (int64_t)blockIdx.x * READ_BLOCK;
  const int nb = (int)(nbytes - b0 < READ_BLOCK ? nbytes - b0 : READ_BLOCK);
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < READ_BLOCK / (WG * 16); ++u) {
    const int ub = u * WG * 16;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p + b0 + ub), (short)0, max(nb - ub, 0), 0x00020000);
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)threadIdx.x * 16, 0, CPOL_NT);
    x ^= (w[0] ^ w[1]) ^ (w[2] ^ w[3]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
  __shared__ uint32_t wx[NWAVE];
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
#pragma unroll
    for (int i = 0; i < NWAVE; ++i) y ^= wx[i];
    if (y == key) out[blockIdx.x] = y;
  }
}

hipError_t launch_read(const void* p, int64_t nbytes, uint32_t key, uint32_t* out, unsigned grid, hipStream_t s) {
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(WG), 0, s, (const char*)p, nbytes, key, out);
  return hipGetLastError();
}

hipError_t launch_probs(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s) {
  KFn f = dtype == D_BF16 ? pick_probs<D_BF16>(mode) : pick_probs<D_F32>(mode);
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

}  // namespace sv

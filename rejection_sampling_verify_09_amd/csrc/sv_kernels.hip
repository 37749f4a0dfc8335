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
//                   chunk once from HBM with 16-byte loads into registers,
//                   and produces the chunk max, sum exp((x - max) / T) and
//                   the filter candidates.  The last chunk of a row to finish
//                   merges the row (max, normaliser, top-k / top-p threshold,
//                   kept list, probability of the drafted token); the last
//                   row of a sequence to finish runs the accept tests, the
//                   first-rejection scan and, for filtered and greedy rows,
//                   the final draw.
//   sample_kernel   unfiltered rows only: the final draw needs the whole
//                   residual / bonus row.  One workgroup per (sequence,
//                   2048-logit chunk) computes the weights in double and their
//                   per-segment sums; the last one scans the segment sums,
//                   finds the segment holding u*Z and rescans it.
//   probs_kernel    writes full filtered rows (sv_filtered_probs).
#include "sv_common.hpp"

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
__device__ __forceinline__ void build_exp_tab(double* tab) {
  __syncthreads();
  if (threadIdx.x < 64) tab[threadIdx.x] = exp2((double)threadIdx.x / 64.0);
  __syncthreads();
}

struct DrawRow {
  double snorm;
  float m;
  uint32_t tau;
};

struct SmemStream {
  uint64_t cand[NWAVE * CAND_CAP];  // per-wave candidate lists (one flat list after an overflow cut)
  uint64_t tk[WG];
  uint32_t hist[256];
  int32_t wn[NWAVE];
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
    double scan[WG];
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
template <int DT>
__device__ uint32_t row_radix(const char* rp, int V, uint32_t lo, bool mass, float m, double invT, double snorm,
                              double target, Smem& sm) {
  const int t = threadIdx.x;
  const unsigned long long tgt = mass ? (unsigned long long)(target * MASS_SCALE) : (unsigned long long)target;
  uint32_t prefix = 0, pmask = 0;
  unsigned long long above = 0;  // F of everything in higher bins at the levels fixed so far
  for (int shift = 24; shift >= 0; shift -= 8) {
    __syncthreads();
    for (int d = t; d < 256; d += WG) sm.r.hist64[d] = 0ull;
    __syncthreads();
    for (int j = t; j < V; j += WG) {
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
template <int DT>
__device__ int row_keep(const char* rp, int V, uint32_t tau, float m, double invT, double* skept, Smem& sm) {
  const int t = threadIdx.x;
  __syncthreads();
  if (t == 0) sm.ncand = 0;
  __syncthreads();
  double acc = 0.0;
  for (int j = t; j < V; j += WG) {
    const float x = load_elem<DT>(rp, j);
    const uint32_t key = ord_key(x);
    if (key >= tau) {
      acc += exp_tab(((double)x - (double)m) * invT, sm.etab);
      const int slot = atomicAdd(&sm.ncand, 1);
      if (slot < KEEP_CAP) sm.r.keys[slot] = ((uint64_t)key << 32) | (uint32_t)j;
    }
  }
  *skept = block_sum(acc, sm.red);
  return sm.ncand;
}

// Radix select (8 bits per pass, counts in LDS) of the k-th largest key among
// the n candidates in sm.r.cand.
__device__ uint32_t cand_select(int n, int k, Smem& sm) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    __syncthreads();
    for (int d = t; d < 256; d += WG) sm.r.hist[d] = 0;
    __syncthreads();
    for (int e = t; e < n; e += WG) {
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
  int off = 0;
  for (int i = 0; i < w; ++i) off += r.i[i];
  *total = ((r.i[0] + r.i[1]) + r.i[2]) + r.i[3];
  return x + off - v;
}

// Sort the first n entries of sm.r.keys descending (pads with zeros).
__device__ void sort_keys_desc(int n, Smem& sm) {
  const int np2 = pow2_at_least(n < 2 ? 2 : n);
  __syncthreads();
  for (int e = n + threadIdx.x; e < np2; e += WG) sm.r.keys[e] = 0;
  bitonic_desc(sm.r.keys, np2);
}

// Top-k / top-p threshold of one row and its kept list.  On entry the chunk
// records are in sm.r (cm, cb, cn) and the row is valid (finite max m;
// for top-p also a finite normaliser rr.S).
template <int DT, int MODE>
__device__ void filter_row(const Args& a, int rl, const char* rp, float m, RowRec& rr, Smem& sm) {
  const int t = threadIdx.x, nch = a.nchunks;
  const uint64_t* cand = a.cand + (size_t)rl * nch * CAND_CAP;
  const double invT = a.invT;

  // Every finite logit with key >= lo is among the candidates: each chunk
  // emitted all of its finite logits at or above its own bound, and lo is the
  // largest bound (and, for top-p, at least the window below the row max).
  uint32_t lo = block_max_u(t < nch ? sm.r.cb[t] : 0u, sm.red);
  if (MODE == M_TOPP) lo = max(lo, ord_key(m - a.win));
  int ncand_total;
  const int my_off = block_excl_scan_i(t < nch ? sm.r.cn[t] : 0, sm.red, &ncand_total);
  if (t < nch) sm.r.off[t] = my_off;
  if (t == 0) sm.r.off[nch] = ncand_total;
  __syncthreads();

  uint32_t tau = 0;
  int nk = 0;          // kept entries held in sm.r.keys, sorted descending
  bool big = false;    // kept set larger than KEEP_CAP
  double skept = 0.0;  // normaliser over the kept set (when big)
  bool fb = ncand_total > ROW_LOAD_MAX;

  if (!fb) {
    // Candidates at or above lo, read in batches of LOAD_BATCH loads per
    // thread: top-p gathers them straight into sm.r.keys (at most KEEP_CAP),
    // top-k into sm.r.cand (at most ROW_CAND) for the radix select.
    uint64_t* dstv = (MODE == M_TOPP) ? sm.r.keys : sm.r.cand;
    const int cap = (MODE == M_TOPP) ? KEEP_CAP : ROW_CAND;
    if (t == 0) sm.ncand = 0;
    __syncthreads();
    for (int base = 0; base < ncand_total; base += WG * LOAD_BATCH) {
      uint64_t ck[LOAD_BATCH];
#pragma unroll
      for (int j = 0; j < LOAD_BATCH; ++j) {
        const int e = base + t + j * WG;
        ck[j] = 0ull;
        if (e < ncand_total) {
          int lo_c = 0, hi_c = nch;  // last chunk with off <= e
          while (hi_c - lo_c > 1) {
            const int mid = (lo_c + hi_c) >> 1;
            if (sm.r.off[mid] <= e) lo_c = mid;
            else hi_c = mid;
          }
          ck[j] = ld_dev(&cand[(size_t)lo_c * CAND_CAP + (e - sm.r.off[lo_c])]);
        }
      }
#pragma unroll
      for (int j = 0; j < LOAD_BATCH; ++j) {
        if (ck[j] != 0ull && (uint32_t)(ck[j] >> 32) >= lo) {
          const int slot = atomicAdd(&sm.ncand, 1);
          if (slot < cap) dstv[slot] = ck[j];
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
        const uint32_t tk = cnt < a.top_k ? KEY_NEG_INF : cand_select(cnt, a.top_k, sm);
        tau = tk;
        // kept set: candidates with key >= tk, into sm.r.keys
        __syncthreads();
        if (t == 0) sm.i1 = 0;
        __syncthreads();
        double sacc = 0.0;
        for (int e = t; e < cnt; e += WG) {
          const uint64_t ce = sm.r.cand[e];
          const uint32_t key = (uint32_t)(ce >> 32);
          if (key >= tk) {
            sacc += exp(((double)key_val(key) - (double)m) * invT);
            const int slot = atomicAdd(&sm.i1, 1);
            if (slot < KEEP_CAP) sm.r.keys[slot] = ce;
          }
        }
        const double sk = block_sum(sacc, sm.red);
        const int nall = sm.i1;
        if (nall <= KEEP_CAP) {
          sort_keys_desc(nall, sm);
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
    } else {  // M_TOPP
      sort_keys_desc(cnt, sm);
      ns = cnt;
    }
    if (!fb && (MODE == M_TOPP || MODE == M_TOPKP)) {
      // smallest descending prefix whose mass reaches top_p, ties included
      const uint32_t key = t < ns ? (uint32_t)(sm.r.keys[t] >> 32) : 0u;
      const double w = t < ns ? exp(((double)key_val(key) - (double)m) * invT) / snorm : 0.0;
      double tot;
      const double C = block_incl_scan(w, sm.red, &tot);
      int first = (t < ns && C >= a.top_p) ? t : INT_MAX;
      first = block_min_i(first, sm.red);
      if (first == INT_MAX) {
        if (MODE == M_TOPP) fb = true;  // the nucleus reaches below the candidate window
        else first = ns - 1;             // round-off kept the top-k mass just below top_p
      }
      if (!fb) {
        if (first < 0) first = 0;
        __syncthreads();
        const uint32_t tp = (uint32_t)(sm.r.keys[first] >> 32);
        tau = tp > tau ? tp : tau;
        nk = block_sum_i((t < ns && key >= tau) ? 1 : 0, sm.red);
      }
    }
  }

  if (fb) {
    // exact cut by a radix search over the whole row (slow, rare)
    rr.flags |= RF_FALLBACK;
    build_exp_tab(sm.etab);
    uint32_t tk = 0;
    double sk = 0.0;
    if (MODE == M_TOPK || MODE == M_TOPKP) {
      tk = row_radix<DT>(rp, a.V, 0u, false, m, invT, 1.0, (double)a.top_k, sm);
      if (MODE == M_TOPKP) (void)row_keep<DT>(rp, a.V, tk, m, invT, &sk, sm);
    }
    if (MODE == M_TOPP || MODE == M_TOPKP) {
      const double sn = MODE == M_TOPP ? rr.S : sk;
      tau = row_radix<DT>(rp, a.V, tk, true, m, invT, sn, a.top_p, sm);
    } else {
      tau = tk;
    }
    const int nall = row_keep<DT>(rp, a.V, tau, m, invT, &skept, sm);
    if (nall <= KEEP_CAP) {
      sort_keys_desc(nall, sm);
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
    skept = block_sum(ex, sm.red);
    // kept list in ascending vocabulary order: re-key as (~index << 32 | key)
    __syncthreads();
    if (t < nk) sm.r.keys[t] = ((uint64_t)(~(uint32_t)e) << 32) | key;
    sort_keys_desc(nk, sm);
    __syncthreads();
    if (t < nk) {
      const uint64_t f = sm.r.keys[t];
      const int idx = (int)~(uint32_t)(f >> 32);
      const float x = key_val((uint32_t)f);
      st_dev(&a.kidx[(size_t)rl * KEEP_CAP + t], idx);
      st_dev(&a.kprob[(size_t)rl * KEEP_CAP + t], exp(((double)x - (double)m) * invT) / skept);
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

template <int DT, int MODE>
__device__ void row_finalize(const Args& a, int rl, int xtok, Smem& sm) {
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
  if (t == WG - 1) sm.lx = (MODE != M_GREEDY && hx) ? load_elem<DT>(rp, xtok) : -INFINITY;
  __syncthreads();
  const float m = block_fmax(t < nch ? sm.r.cm[t] : -INFINITY, sm.red);
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
    const double s = qm > -INFINITY ? sm.r.cs[t] * exp(((double)qm - (double)m) * a.invT) : 0.0;
    const double S = block_sum(s, sm.red);
    rr.S = S;
    if (!(S > 0.0 && S < INFINITY)) bad = true;
  }
  if (MODE == M_GREEDY) {
    const int best = block_min_i((t < nch && sm.r.cm[t] == m) ? sm.r.carg[t] : INT_MAX, sm.red);
    rr.arg = best == INT_MAX ? 0 : best;
  }
  if (FILT) {
    if (!bad) filter_row<DT, MODE>(a, rl, rp, m, rr, sm);
  }
  if (!bad && hx) {
    if (MODE == M_GREEDY) {
      rr.px = xtok == rr.arg ? 1.0 : 0.0;
    } else {
      const float lx = sm.lx;
      if (ord_key(lx) >= rr.tau) rr.px = exp(((double)lx - (double)m) * a.invT) / (MODE == M_PLAIN ? rr.S : rr.S_kept);
    }
  }
  if (bad) rr.flags |= RF_BAD;
  __syncthreads();
  if (t == 0) store_row(&a.row[rl], rr);
}

// ---------------------------------------------------------------------------
// final draw
// ---------------------------------------------------------------------------

// Draw from the kept lists (filtered rows): residual max(0, p - q) over the
// target's kept tokens, or p itself (bonus, or an empty residual).
__device__ int list_sample(const Args& a, double u, int rlP, int np, int rlQ, int nq, bool res, Smem& sm,
                           double* Zout) {
  const int t = threadIdx.x;
  __syncthreads();
  if (t < np) {
    sm.q.pidx[t] = ld_dev(&a.kidx[(size_t)rlP * KEEP_CAP + t]);
    sm.q.pprob[t] = ld_dev(&a.kprob[(size_t)rlP * KEEP_CAP + t]);
  }
  if (res && t < nq) {
    sm.q.qidx[t] = ld_dev(&a.kidx[(size_t)rlQ * KEEP_CAP + t]);
    sm.q.qprob[t] = ld_dev(&a.kprob[(size_t)rlQ * KEEP_CAP + t]);
  }
  __syncthreads();
  double p = 0.0, w = 0.0;
  if (t < np) {
    p = sm.q.pprob[t];
    w = p;
    if (res) {
      const int idx = sm.q.pidx[t];
      int lo = 0, hi = nq;  // first position with qidx >= idx
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sm.q.qidx[mid] < idx) lo = mid + 1;
        else hi = mid;
      }
      const double q = (lo < nq && sm.q.qidx[lo] == idx) ? sm.q.qprob[lo] : 0.0;
      const double d = p - q;
      w = d > 0.0 ? d : 0.0;
    }
  }
  double Z;
  double C = block_incl_scan(w, sm.red, &Z);
  if (res && !(Z > 0.0)) {
    w = p;
    C = block_incl_scan(w, sm.red, &Z);
  }
  const double target = u * Z;
  int first = (t < np && target < C) ? t : INT_MAX;
  first = block_min_i(first, sm.red);
  if (first == INT_MAX) first = block_max_i((t < np && w > 0.0) ? t : -1, sm.red);
  if (first < 0) first = 0;
  *Zout = Z;
  return sm.q.pidx[first];
}

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
                                              double invT, const double* tab) {
  const float xp = load_elem<DT>(pr, j);
  double w = ord_key(xp) >= dr[0].tau ? exp_tab(((double)xp - (double)dr[0].m) * invT, tab) / dr[0].snorm : 0.0;
  if (use_res) {
    const float xq = load_elem<DT>(qr, j);
    const double q = ord_key(xq) >= dr[1].tau ? exp_tab(((double)xq - (double)dr[1].m) * invT, tab) / dr[1].snorm : 0.0;
    const double d = w - q;
    w = d > 0.0 ? d : 0.0;
  }
  return w;
}

template <int DT>
__device__ int full_row_sample(const Args& a, double u, const char* pr, const char* qr, bool res, Smem& sm,
                               double* Zout) {
  const int t = threadIdx.x, V = a.V;
  const double invT = a.invT;
  const DrawRow* dr = sm.dr;
  build_exp_tab(sm.etab);
  bool use_res = res;
  double Z = 0.0;
  int lastpos = -1;
  for (int pass = 0; pass < 2; ++pass) {
    Z = 0.0;
    lastpos = -1;
    for (int base = 0; base < V; base += SCE) {
      double ts = 0.0;
#pragma unroll 1
      for (int e = 0; e < 8; ++e) {
        const int j = base + t * 8 + e;
        if (j < V) {
          const double w = draw_weight<DT>(pr, qr, j, dr, use_res, invT, sm.etab);
          ts += w;
          if (w > 0.0) lastpos = j;
        }
      }
      Z += block_sum(ts, sm.red);
    }
    lastpos = block_max_i(lastpos, sm.red);
    if (!use_res || Z > 0.0) break;
    use_res = false;  // empty residual: draw from p
  }
  const double target = u * Z;
  double run = 0.0;
  int tok = -1;
  for (int base = 0; base < V && tok < 0; base += SCE) {
    double ts = 0.0;
#pragma unroll 1
    for (int e = 0; e < 8; ++e) {
      const int j = base + t * 8 + e;
      if (j < V) ts += draw_weight<DT>(pr, qr, j, dr, use_res, invT, sm.etab);
    }
    const double tile = block_sum(ts, sm.red);
    if (run + tile > target) {
      double tot;
      const double incl = block_incl_scan(ts, sm.red, &tot);
      __syncthreads();
      sm.scan[t] = incl;
      __syncthreads();
      double C = run + (t > 0 ? sm.scan[t - 1] : 0.0);
      int first = INT_MAX, lastp = -1;
#pragma unroll 1
      for (int e = 0; e < 8; ++e) {
        const int j = base + t * 8 + e;
        if (j < V) {
          const double w = draw_weight<DT>(pr, qr, j, dr, use_res, invT, sm.etab);
          C += w;
          if (w > 0.0) {
            lastp = j;
            if (first == INT_MAX && target < C) first = j;
          }
        }
      }
      first = block_min_i(first, sm.red);
      tok = first != INT_MAX ? first : block_max_i(lastp, sm.red);
    }
    run += tile;
  }
  if (tok < 0) tok = lastpos < 0 ? 0 : lastpos;
  *Zout = Z;
  return tok;
}

// Parameters of a row for the full-row draw, into sm.dr[slot].
__device__ __forceinline__ void set_draw_row(const RowRec* r, bool filtered, int slot, Smem& sm) {
  __syncthreads();
  if (threadIdx.x == 0) {
    sm.dr[slot].m = ld_dev(&r->m);
    sm.dr[slot].tau = ld_dev(&r->tau);
    sm.dr[slot].snorm = filtered ? ld_dev(&r->S_kept) : ld_dev(&r->S);
  }
  __syncthreads();
}

template <int DT, int MODE>
__device__ void seq_finalize(const Args& a, int b, Smem& sm) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x, K = a.K, rps = a.rps;
  const RowRec* rr = a.row + (size_t)b * rps;
  __syncthreads();
  // one round trip: row records, drafted tokens and uniforms
  if (t < rps) {
    sm.q.px[t] = ld_dev(&rr[t].px);
    sm.q.rf[t] = ld_dev(&rr[t].flags);
    if (MODE == M_GREEDY) sm.q.arg[t] = ld_dev(&rr[t].arg);
    else sm.q.nk[t] = ld_dev(&rr[t].nkept);
  }
  if (t < K) sm.q.x[t] = a.X[(size_t)b * K + t];
  if (t <= K) sm.q.u[t] = a.U[(size_t)b * (K + 1) + t];
  __syncthreads();
  if (t == 0) {
    int bad = 0;
    for (int j = 0; j < rps; ++j) bad |= sm.q.rf[j] & RF_BAD;
    for (int i = 0; i < K; ++i)
      if (sm.q.x[i] < 0 || sm.q.x[i] >= a.V) bad = 1;
    int n = K;
    for (int i = 0; i < K; ++i) {
      const double p = sm.q.px[i];
      const bool acc = MODE == M_GREEDY ? p > 0.0 : (double)sm.q.u[i] * sm.q.px[K + 1 + i] < p;
      if (!acc) {
        n = i;
        break;
      }
    }
    sm.i0 = bad ? -1 : n;
  }
  __syncthreads();
  const int n = sm.i0;
  int32_t* ot = a.out_tok + (size_t)b * (K + 1);
  if (a.out_p || a.out_q) {
    const double nanv = __longlong_as_double(0x7FF8000000000000ll);
    for (int i = t; i < K; i += WG) {
      if (a.out_p) a.out_p[(size_t)b * K + i] = n < 0 ? nanv : sm.q.px[i];
      if (a.out_q) a.out_q[(size_t)b * K + i] = (n < 0 || MODE == M_GREEDY) ? nanv : sm.q.px[K + 1 + i];
    }
  }
  if (n < 0) {
    for (int j = t; j <= K; j += WG) ot[j] = -1;
    if (t == 0) {
      a.out_n[b] = -1;
      SeqRec s;
      s.Z = 0.0;
      s.n = -1;
      s.flags = RF_BAD;
      a.seq[b] = s;
      if (a.out_z) a.out_z[b] = __longlong_as_double(0x7FF8000000000000ll);
    }
    return;
  }
  for (int j = t; j <= K; j += WG) {
    if (j < n) ot[j] = sm.q.x[j];
    else if (j > n) ot[j] = -1;
  }
  if (t == 0) a.out_n[b] = n;
  if (MODE == M_PLAIN) {
    if (t == 0) {
      SeqRec s;
      s.Z = 0.0;
      s.n = n;
      s.flags = 0;
      a.seq[b] = s;
    }
    return;  // the sampling kernel draws the last token
  }
  int tok;
  double Z = 1.0;
  if (MODE == M_GREEDY) {
    tok = sm.q.arg[n];
  } else {
    const double u = (double)sm.q.u[K];
    const bool res = n < K;
    const int jq = res ? K + 1 + n : n;
    const int rlP = b * rps + n, rlQ = b * rps + jq;
    const int np = sm.q.nk[n], nq = sm.q.nk[jq];
    if (np < 0 || (res && nq < 0)) {
      set_draw_row(&rr[n], true, 0, sm);
      set_draw_row(&rr[jq], true, 1, sm);
      tok = full_row_sample<DT>(a, u, row_ptr(a, rlP, ESZ), row_ptr(a, rlQ, ESZ), res, sm, &Z);
    } else {
      tok = list_sample(a, u, rlP, np, rlQ, nq, res, sm, &Z);
    }
  }
  if (t == 0) {
    ot[n] = tok;
    if (a.out_z) a.out_z[b] = Z;
  }
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// Append every logit of this thread at or above thr to its wave's candidate
// list wl (entries ord_key << 32 | index, slots past CAND_CAP dropped) and
// return the wave's count.  Compaction by ballot: a register slot costs one
// compare and a scalar branch unless some lane of the wave qualifies.  Called
// with every lane of the wave active.
template <int DT, bool VEC>
__device__ __forceinline__ int wave_emit(const float (&v)[EPT], float tm, float thr, int c0, uint64_t* wl) {
  int wn = 0;
  if (__ballot(tm >= thr) == 0ull) return 0;
#pragma unroll
  for (int k = 0; k < EPT; ++k) {
    const bool pr = v[k] >= thr;
    const unsigned long long bm = __ballot(pr);
    if (bm != 0ull) {
      if (pr) {
        const int pos =
            wn + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
        if (pos < CAND_CAP)
          wl[pos] = ((uint64_t)ord_key(v[k]) << 32) | (uint32_t)(c0 + local_index<DT, VEC>(k, threadIdx.x));
      }
      wn += __popcll(bm);
    }
  }
  return wn;
}

// One chunk item: stream it and leave its record (max, sum, candidates).
template <int DT, int MODE, bool VEC>
__device__ __forceinline__ void stream_item(const Args& a, int item, Smem& sm) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  constexpr bool FILT = MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP;
  const int t = threadIdx.x;
  const int rl = item / a.nchunks;
  const int c = item - rl * a.nchunks;
  const int chunk_id = item;
  const char* rp = row_ptr(a, rl, ESZ);
  const int c0 = c * CE, cn = min(CE, a.V - c0);

  float v[EPT];
  load_chunk<DT, VEC>(rp, c0, cn, v);
  // maxima of 4 groups of 8 register slots, then of the thread
  float gm[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float x = v[8 * g];
#pragma unroll
    for (int e = 1; e < 8; ++e) x = fmaxf(x, v[8 * g + e]);
    gm[g] = x;
  }
  const float tm = fmaxf(fmaxf(gm[0], gm[1]), fmaxf(gm[2], gm[3]));
  if (t == 0) sm.ncand = 0;
  const float mc = block_fmax(tm, sm.red);

  ChunkRec rec;
  rec.s = 0.0;
  rec.m = mc;
  rec.bound = 0u;
  rec.ncand = 0;
  rec.arg = 0;
  rec.pad0 = rec.pad1 = 0;

  // candidate bound of this chunk: every finite logit at or above it is emitted
  uint32_t bound = 0u;
  float thr = 0.0f;
  if (FILT) {
    if (MODE == M_TOPP) {
      // window below the chunk max (which is <= the row max)
      bound = ord_key(mc - a.win);
    } else {
      // the k-th largest of the 256 thread maxima is <= the row's k-th largest
      // logit (for k > 256 no bound follows: every finite logit qualifies)
      sm.s.tk[t] = ord_key(tm);
      bitonic_desc(sm.s.tk, WG);
      bound = a.top_k <= WG ? (uint32_t)sm.s.tk[a.top_k - 1] : KEY_NEG_INF;
    }
    thr = bound > KEY_NEG_INF ? key_val(bound) : -3.402823466e38f;
  }
  if (MODE == M_PLAIN || MODE == M_TOPP) {
    // sum of exp2((x - mc) * c2): one fma per logit against M = fl(mc * c2);
    // the (exactly known) rounding of M is a common factor fixed once per
    // chunk.
    float acc = 0.0f;
    double corr = 1.0;
    if (mc > -INFINITY) {
      const float c2 = a.c2;
      const float M = mc * c2;
      if (M > -INFINITY && M < INFINITY) {
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          acc += __builtin_amdgcn_exp2f(__builtin_fmaf(v[k], c2, -M));
        }
        corr = exp2((double)M - (double)mc * (double)c2);
      } else {
#pragma unroll
        for (int k = 0; k < EPT; ++k) {
          acc += __builtin_amdgcn_exp2f((v[k] - mc) * c2);
        }
      }
    }
    rec.s = block_sum((double)acc, sm.red) * corr;
  }

  if (MODE == M_GREEDY) {
    int best = INT_MAX;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (v[k] == mc) best = min(best, local_index<DT, VEC>(k, t));
    best = block_min_i(best, sm.red);
    rec.arg = c0 + (best == INT_MAX ? 0 : best);
  }

  if (FILT) {
    const int w = t >> 6;
    const int wn = wave_emit<DT, VEC>(v, tm, thr, c0, &sm.s.cand[w * CAND_CAP]);
    if ((t & 63) == 0) sm.s.wn[w] = wn;
    __syncthreads();
    int nc = (sm.s.wn[0] + sm.s.wn[1]) + (sm.s.wn[2] + sm.s.wn[3]);
    uint64_t* dst = a.cand + (size_t)chunk_id * CAND_CAP;
    if (nc <= CAND_CAP) {
      int off = 0;
      for (int i = 0; i < w; ++i) off += sm.s.wn[i];
      for (int s = t & 63; s < wn; s += 64) st_dev(&dst[off + s], sm.s.cand[w * CAND_CAP + s]);
    } else {
      // Too many: keep exactly the candidates above the (CAND_CAP+1)-th largest
      // key (radix select over the registers) and raise the bound to match.
      uint32_t prefix = 0, pmask = 0;
      int need = CAND_CAP + 1;
      for (int shift = 24; shift >= 0; shift -= 8) {
        __syncthreads();
        sm.s.hist[t] = 0u;
        __syncthreads();
        for (int g = 0; g < 4; ++g) {
          if (gm[g] >= thr) {
            float wv[8];
            load_group<DT, VEC>(rp, c0, cn, g, wv);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t key = ord_key(wv[e]);
              if (wv[e] >= thr && (key & pmask) == prefix) atomicAdd(&sm.s.hist[(key >> shift) & 255u], 1u);
            }
          }
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
      bound = prefix + 1u;  // every candidate with key >= bound fits
      for (int g = 0; g < 4; ++g) {
        if (gm[g] >= thr) {
          float wv[8];
          load_group<DT, VEC>(rp, c0, cn, g, wv);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t key = ord_key(wv[e]);
            if (wv[e] >= thr && key >= bound) {
              const int s2 = atomicAdd(&sm.ncand, 1);
              if (s2 < CAND_CAP)
                sm.s.cand[s2] = ((uint64_t)key << 32) | (uint32_t)(c0 + local_index<DT, VEC>(8 * g + e, t));
            }
          }
        }
      }
      __syncthreads();
      nc = sm.ncand;
      for (int s = t; s < nc; s += WG) st_dev(&dst[s], sm.s.cand[s]);
    }
    rec.ncand = nc;
    rec.bound = bound;
  }
  if (t == 0) {
    ChunkRec* cp = &a.chunk[chunk_id];
    if (MODE == M_PLAIN || MODE == M_TOPP) st_dev(&cp->s, rec.s);
    st_dev(&cp->m, rec.m);
    if (FILT) {
      st_dev(&cp->bound, rec.bound);
      st_dev(&cp->ncand, rec.ncand);
    }
    if (MODE == M_GREEDY) st_dev(&cp->arg, rec.arg);
  }

}

// One workgroup per (row, chunk).  No workgroup waits on another: the row
// merge runs in the next launch, when HBM is no longer saturated and its few
// dependent round trips are short.
template <int DT, int MODE, bool VEC>
__global__ void __launch_bounds__(WG, STREAM_WG_PER_CU) stream_kernel(Args a) {
  __shared__ Smem sm;
  stream_item<DT, MODE, VEC>(a, (int)blockIdx.x, sm);
}

// One workgroup per row: merge the chunk records into the row's max,
// normaliser, filter threshold, kept list and the probability of its drafted
// token; the last row of a sequence to finish runs the accept tests, the
// first-rejection scan and (filtered and greedy rows) the final draw.
template <int DT, int MODE>
__global__ void __launch_bounds__(WG) row_kernel(Args a) {
  __shared__ Smem sm;
  const int rl = (int)blockIdx.x;
  const int b = rl / a.rps, jr = rl - b * a.rps;
  const int ir = jr <= a.K ? jr : jr - a.K - 1;
  const int xtok = (a.do_seq && ir < a.K) ? a.X[(size_t)b * a.K + ir] : -1;
  row_finalize<DT, MODE>(a, rl, xtok, sm);
  if (a.do_seq && last_arrival(&a.seq_cnt[b], (uint32_t)a.rps, &sm.flag)) seq_finalize<DT, MODE>(a, b, sm);
}

template <int DT>
__device__ __forceinline__ double plain_weight(const char* pr, const char* qr, int j, const RowRec& P,
                                               const RowRec& Q, bool res, double invT) {
  const double p = exp(((double)load_elem<DT>(pr, j) - (double)P.m) * invT) / P.S;
  if (!res) return p;
  const double q = exp(((double)load_elem<DT>(qr, j) - (double)Q.m) * invT) / Q.S;
  const double d = p - q;
  return d > 0.0 ? d : 0.0;
}

template <int DT>
__global__ void __launch_bounds__(WG) sample_kernel(Args a) {
  __shared__ Smem sm;
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x;
  const int b = (int)(blockIdx.x / (unsigned)a.nsc);
  const int c = (int)blockIdx.x - b * a.nsc;
  const int K = a.K;
  const int nseg = a.nsc * SEG_PER_SCE;
  const SeqRec sr = a.seq[b];
  const int n = sr.n;
  const bool active = n >= 0;
  const bool res = active && n < K;
  const int rlP = b * a.rps + (active ? n : 0);
  const int rlQ = b * a.rps + (res ? K + 1 + n : (active ? n : 0));
  RowRec P, Q;
  const char* pr = nullptr;
  const char* qr = nullptr;
  if (active) {
    P = a.row[rlP];
    Q = a.row[rlQ];
    pr = row_ptr(a, rlP, ESZ);
    qr = row_ptr(a, rlQ, ESZ);
    const int j0 = c * SCE + t * 8;
    double ts = 0.0;
    int lastp = -1;
    for (int e = 0; e < 8; ++e) {
      const int j = j0 + e;
      if (j < a.V) {
        const double w = plain_weight<DT>(pr, qr, j, P, Q, res, a.invT);
        ts += w;
        if (w > 0.0) lastp = j;
      }
    }
    const double ss = wave_sum(ts);
    const int sl = wave_max(lastp);
    if ((t & 63) == 0) {
      const size_t s = (size_t)b * nseg + c * SEG_PER_SCE + (t >> 6);
      st_dev(&a.seg_sum[s], ss);
      st_dev(&a.seg_last[s], sl);
    }
  }
  if (!last_arrival(&a.smp_cnt[b], (uint32_t)a.nsc, &sm.flag)) return;
  if (!active) return;

  const double* ssum = a.seg_sum + (size_t)b * nseg;
  const int32_t* slast = a.seg_last + (size_t)b * nseg;
  const int per = (nseg + WG - 1) / WG;
  const int s0 = min(t * per, nseg), s1 = min(s0 + per, nseg);
  double loc = 0.0;
  int lastseg = -1;
  for (int s = s0; s < s1; ++s) {
    loc += ld_dev(&ssum[s]);
    if (ld_dev(&slast[s]) >= 0) lastseg = s;
  }
  double Z;
  const double incl = block_incl_scan(loc, sm.red, &Z);
  lastseg = block_max_i(lastseg, sm.red);
  const double u = (double)a.U[(size_t)b * (K + 1) + K];
  int tok;
  if (!(Z > 0.0)) {
    // empty residual (round-off only): draw from p
    set_draw_row(&a.row[rlP], false, 0, sm);
    tok = full_row_sample<DT>(a, u, pr, qr, false, sm, &Z);
  } else {
    const double target = u * Z;
    __syncthreads();
    sm.scan[t] = incl;
    __syncthreads();
    double run = t > 0 ? sm.scan[t - 1] : 0.0;
    int found = INT_MAX;
    double cstart = 0.0;
    for (int s = s0; s < s1; ++s) {
      const double ce = run + ld_dev(&ssum[s]);
      if (found == INT_MAX && target < ce) {
        found = s;
        cstart = run;
      }
      run = ce;
    }
    const int sf = block_min_i(found, sm.red);
    if (sf == INT_MAX) {
      tok = lastseg >= 0 ? ld_dev(&slast[lastseg]) : 0;
    } else {
      __syncthreads();
      if (found == sf) sm.d0 = cstart;
      __syncthreads();
      const double cs = sm.d0;
      const int j0 = sf * SEG + 2 * t;
      const double w0 = j0 < a.V ? plain_weight<DT>(pr, qr, j0, P, Q, res, a.invT) : 0.0;
      const double w1 = j0 + 1 < a.V ? plain_weight<DT>(pr, qr, j0 + 1, P, Q, res, a.invT) : 0.0;
      double tot;
      const double inc2 = block_incl_scan(w0 + w1, sm.red, &tot);
      __syncthreads();
      sm.scan[t] = inc2;
      __syncthreads();
      const double C0 = cs + (t > 0 ? sm.scan[t - 1] : 0.0) + w0;
      const double C1 = C0 + w1;
      int first = INT_MAX;
      if (j0 < a.V && w0 > 0.0 && target < C0) first = j0;
      else if (j0 + 1 < a.V && w1 > 0.0 && target < C1) first = j0 + 1;
      first = block_min_i(first, sm.red);
      tok = first != INT_MAX ? first : ld_dev(&slast[sf]);
      if (tok < 0) tok = lastseg >= 0 ? ld_dev(&slast[lastseg]) : 0;
    }
  }
  if (t == 0) {
    a.out_tok[(size_t)b * (K + 1) + n] = tok;
    if (a.out_z) a.out_z[b] = Z;
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
      else out = (float)kept_prob<DT>(rp, j, R, filtered, a.invT);
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
  return vec ? (KFn)stream_kernel<DT, MODE, true> : (KFn)stream_kernel<DT, MODE, false>;
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

template <int DT>
static KFn pick_row(int mode) {
  switch (mode) {
    case M_PLAIN: return (KFn)row_kernel<DT, M_PLAIN>;
    case M_TOPK: return (KFn)row_kernel<DT, M_TOPK>;
    case M_TOPP: return (KFn)row_kernel<DT, M_TOPP>;
    case M_TOPKP: return (KFn)row_kernel<DT, M_TOPKP>;
    default: return (KFn)row_kernel<DT, M_GREEDY>;
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

hipError_t launch_stream(const Args& a, int dtype, int mode, bool vec, unsigned grid, hipStream_t s) {
  KFn f = dtype == D_BF16 ? pick_stream_mode<D_BF16>(mode, vec) : pick_stream_mode<D_F32>(mode, vec);
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_row(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s) {
  KFn f = dtype == D_BF16 ? pick_row<D_BF16>(mode) : pick_row<D_F32>(mode);
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sample(const Args& a, int dtype, unsigned grid, hipStream_t s) {
  KFn f = dtype == D_BF16 ? (KFn)sample_kernel<D_BF16> : (KFn)sample_kernel<D_F32>;
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_probs(const Args& a, int dtype, int mode, unsigned grid, hipStream_t s) {
  KFn f = dtype == D_BF16 ? pick_probs<D_BF16>(mode) : pick_probs<D_F32>(mode);
  hipLaunchKernelGGL(f, dim3(grid), dim3(WG), 0, s, a);
  return hipGetLastError();
}

}  // namespace sv

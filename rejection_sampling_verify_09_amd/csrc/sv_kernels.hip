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

struct SmemStream {
  uint64_t cand[CAND_CAP];
  uint64_t tk[WG];
};
struct SmemRow {
  uint64_t keys[KEEP_CAP];
  uint32_t hist[256];
};
struct SmemSeq {
  int32_t pidx[KEEP_CAP];
  int32_t qidx[KEEP_CAP];
  double pprob[KEEP_CAP];
  double qprob[KEEP_CAP];
  double px[MAX_RPS];
  int32_t rf[MAX_RPS];
};
struct Smem {
  union {
    SmemStream s;
    SmemRow r;
    SmemSeq q;
    double scan[WG];
  };
  Red red;
  int32_t ncand;
  int32_t flag;
  int32_t i0, i1;
  uint32_t u0;
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

// ---------------------------------------------------------------------------
// row merge helpers
// ---------------------------------------------------------------------------

// F(t) over the whole row: number of logits with key >= max(t, lo), or their
// probability mass exp((x - m) / T) / snorm.
template <int DT>
__device__ double row_F(const char* rp, int V, uint32_t tk, uint32_t lo, bool mass, float m, double invT,
                        double snorm, Smem& sm) {
  const uint32_t th = tk > lo ? tk : lo;
  double acc = 0.0;
  for (int j = threadIdx.x; j < V; j += WG) {
    const float x = load_elem<DT>(rp, j);
    if (ord_key(x) >= th) acc += mass ? exp(((double)x - (double)m) * invT) / snorm : 1.0;
  }
  return block_sum(acc, sm.red);
}

// Largest key t >= lo with F(t) >= target (F is non-increasing in t); this is
// the key of an actual logit, the cut of a top-k (counts) or top-p (mass) set.
template <int DT>
__device__ uint32_t row_bisect(const char* rp, int V, uint32_t lo, bool mass, float m, double invT, double snorm,
                               double target, Smem& sm) {
  uint32_t hi = 0xFFFFFFFFu;
  while (lo < hi) {
    const uint32_t mid = lo + (uint32_t)((((uint64_t)hi - lo) + 1) >> 1);
    if (row_F<DT>(rp, V, mid, lo, mass, m, invT, snorm, sm) >= target)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// k-th largest candidate key among the candidates with key >= lo (radix
// select, 8 bits per pass, counts in LDS).
__device__ uint32_t cand_select(const ChunkRec* cr, const uint64_t* cand, int nch, uint32_t lo, int k, Smem& sm) {
  const int t = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int need = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    __syncthreads();
    for (int d = t; d < 256; d += WG) sm.r.hist[d] = 0;
    __syncthreads();
    for (int p = t; p < nch * CAND_CAP; p += WG) {
      const int c = p / CAND_CAP, s = p - c * CAND_CAP;
      if (s < min(cr[c].ncand, CAND_CAP)) {
        const uint32_t key = (uint32_t)(cand[p] >> 32);
        if (key >= lo && (key & pmask) == prefix) atomicAdd(&sm.r.hist[(key >> shift) & 255u], 1u);
      }
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

// Gather candidates with key >= th into sm.r.keys (value-key << 32 | index);
// returns how many qualified (entries beyond KEEP_CAP are not stored).
__device__ int cand_gather(const ChunkRec* cr, const uint64_t* cand, int nch, uint32_t th, Smem& sm) {
  const int t = threadIdx.x;
  __syncthreads();
  if (t == 0) sm.ncand = 0;
  __syncthreads();
  for (int p = t; p < nch * CAND_CAP; p += WG) {
    const int c = p / CAND_CAP, s = p - c * CAND_CAP;
    if (s < min(cr[c].ncand, CAND_CAP)) {
      const uint64_t e = cand[p];
      if ((uint32_t)(e >> 32) >= th) {
        const int slot = atomicAdd(&sm.ncand, 1);
        if (slot < KEEP_CAP) sm.r.keys[slot] = e;
      }
    }
  }
  __syncthreads();
  return sm.ncand;
}

// Gather every logit of the row with key >= th (full-row pass).
template <int DT>
__device__ int row_gather(const char* rp, int V, uint32_t th, Smem& sm) {
  const int t = threadIdx.x;
  __syncthreads();
  if (t == 0) sm.ncand = 0;
  __syncthreads();
  for (int j = t; j < V; j += WG) {
    const uint32_t key = ord_key(load_elem<DT>(rp, j));
    if (key >= th) {
      const int slot = atomicAdd(&sm.ncand, 1);
      if (slot < KEEP_CAP) sm.r.keys[slot] = ((uint64_t)key << 32) | (uint32_t)j;
    }
  }
  __syncthreads();
  return sm.ncand;
}

// Sort the first n entries of sm.r.keys descending (pads with zeros).
__device__ void sort_keys_desc(int n, Smem& sm) {
  const int np2 = pow2_at_least(n < 2 ? 2 : n);
  __syncthreads();
  for (int e = n + threadIdx.x; e < np2; e += WG) sm.r.keys[e] = 0;
  bitonic_desc(sm.r.keys, np2);
}

// Top-k / top-p threshold of one row and its kept list.  On entry the row is
// valid (finite max m; for top-p also a finite normaliser rr.S).
template <int DT, int MODE>
__device__ void filter_row(const Args& a, int rl, const char* rp, float m, RowRec& rr, Smem& sm) {
  const int t = threadIdx.x, nch = a.nchunks;
  const ChunkRec* cr = a.chunk + (size_t)rl * nch;
  const uint64_t* cand = a.cand + (size_t)rl * nch * CAND_CAP;
  const double invT = a.invT;

  // Every logit with key >= lo is among the candidates (each chunk emitted
  // all its finite logits at or above its own bound, and every bound <= lo),
  // unless a chunk that may hold such logits ran out of slots.
  uint32_t lo;
  if (MODE == M_TOPP) {
    lo = ord_key(m - a.win);
  } else {
    uint32_t mb = 0;
    for (int c = t; c < nch; c += WG) mb = max(mb, cr[c].bound);
    lo = block_max_u(mb, sm.red);
  }
  int spoil = 0;
  for (int c = t; c < nch; c += WG) {
    const ChunkRec q = cr[c];
    if (q.ncand > CAND_CAP && ord_key(q.m) >= lo) spoil = 1;
  }
  spoil = block_max_i(spoil, sm.red);

  uint32_t tau = 0;
  int nk = 0;          // kept entries held in sm.r.keys, sorted descending
  bool big = false;    // kept set larger than KEEP_CAP
  double skept = 0.0;  // normaliser over the kept set (when big)
  bool fb = spoil != 0;

  if (!fb) {
    double snorm = rr.S;  // top-p normaliser
    int ns = 0;           // sorted entries available for the top-p walk
    if (MODE == M_TOPK || MODE == M_TOPKP) {
      int cnt = 0;
      for (int p = t; p < nch * CAND_CAP; p += WG) {
        const int c = p / CAND_CAP, s = p - c * CAND_CAP;
        if (s < min(cr[c].ncand, CAND_CAP) && (uint32_t)(cand[p] >> 32) >= lo) ++cnt;
      }
      cnt = block_sum_i(cnt, sm.red);
      // fewer than k finite logits: every bound was -inf and all of them are kept
      const uint32_t tk = cnt < a.top_k ? KEY_NEG_INF : cand_select(cr, cand, nch, lo, a.top_k, sm);
      const int nall = cand_gather(cr, cand, nch, tk, sm);
      tau = tk;
      if (nall <= KEEP_CAP) {
        sort_keys_desc(nall, sm);
        ns = nall;
        nk = nall;
        if (MODE == M_TOPKP) {
          const double e = t < ns ? exp(((double)key_val((uint32_t)(sm.r.keys[t] >> 32)) - (double)m) * invT) : 0.0;
          snorm = block_sum(e, sm.red);
        }
      } else if (MODE == M_TOPK) {
        big = true;
        double s = 0.0;
        for (int p = t; p < nch * CAND_CAP; p += WG) {
          const int c = p / CAND_CAP, sl = p - c * CAND_CAP;
          if (sl < min(cr[c].ncand, CAND_CAP)) {
            const uint32_t key = (uint32_t)(cand[p] >> 32);
            if (key >= tk) s += exp(((double)key_val(key) - (double)m) * invT);
          }
        }
        skept = block_sum(s, sm.red);
      } else {
        fb = true;  // top-p over a top-k set too large for LDS
      }
    } else {  // M_TOPP
      const int nall = cand_gather(cr, cand, nch, lo, sm);
      if (nall > KEEP_CAP) {
        fb = true;
      } else {
        sort_keys_desc(nall, sm);
        ns = nall;
      }
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
    // exact threshold by bisection over the whole row (slow, rare)
    rr.flags |= RF_FALLBACK;
    uint32_t tk = 0;
    double sk = 0.0;
    if (MODE == M_TOPK || MODE == M_TOPKP) {
      tk = row_bisect<DT>(rp, a.V, 0u, false, m, invT, 1.0, (double)a.top_k, sm);
      sk = row_F<DT>(rp, a.V, tk, 0u, true, m, invT, 1.0, sm);
    }
    if (MODE == M_TOPP || MODE == M_TOPKP) {
      const double sn = MODE == M_TOPP ? rr.S : sk;
      tau = row_bisect<DT>(rp, a.V, tk, true, m, invT, sn, a.top_p, sm);
    } else {
      tau = tk;
    }
    const int nall = (int)row_F<DT>(rp, a.V, tau, 0u, false, m, invT, 1.0, sm);
    if (nall <= KEEP_CAP) {
      row_gather<DT>(rp, a.V, tau, sm);
      sort_keys_desc(nall, sm);
      nk = nall;
    } else {
      big = true;
      skept = row_F<DT>(rp, a.V, tau, 0u, true, m, invT, 1.0, sm);
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
      a.kidx[(size_t)rl * KEEP_CAP + t] = idx;
      a.kprob[(size_t)rl * KEEP_CAP + t] = exp(((double)x - (double)m) * invT) / skept;
    }
  }
  rr.tau = tau;
  rr.S_kept = skept;
  rr.nkept = big ? -1 : nk;
  if (big) rr.flags |= RF_BIG;
}

template <int DT, int MODE>
__device__ void row_finalize(const Args& a, int rl, Smem& sm) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x, nch = a.nchunks;
  const ChunkRec* cr = a.chunk + (size_t)rl * nch;
  const char* rp = row_ptr(a, rl, ESZ);
  float m = -INFINITY;
  for (int c = t; c < nch; c += WG) m = fmaxf(m, cr[c].m);
  m = block_fmax(m, sm.red);
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
    double s = 0.0;
    for (int c = t; c < nch; c += WG) {
      const ChunkRec q = cr[c];
      if (q.m > -INFINITY) s += q.s * exp(((double)q.m - (double)m) * a.invT);
    }
    const double S = block_sum(s, sm.red);
    rr.S = S;
    if (!(S > 0.0 && S < INFINITY)) bad = true;
  }
  if (MODE == M_GREEDY) {
    int best = INT_MAX;
    for (int c = t; c < nch; c += WG)
      if (cr[c].m == m) best = min(best, cr[c].arg);
    best = block_min_i(best, sm.red);
    rr.arg = best == INT_MAX ? 0 : best;
  }
  if (MODE == M_TOPK || MODE == M_TOPP || MODE == M_TOPKP) {
    if (!bad) filter_row<DT, MODE>(a, rl, rp, m, rr, sm);
  }
  const int b = rl / a.rps, j = rl - b * a.rps;
  const int i = j <= a.K ? j : j - a.K - 1;
  if (!bad && i < a.K) {
    const int x = a.X[(size_t)b * a.K + i];
    double px = 0.0;
    if (x >= 0 && x < a.V) {
      if (MODE == M_GREEDY) {
        px = x == rr.arg ? 1.0 : 0.0;
      } else {
        const float lx = load_elem<DT>(rp, x);
        if (ord_key(lx) >= rr.tau) {
          const double e = exp(((double)lx - (double)m) * a.invT);
          px = e / (MODE == M_PLAIN ? rr.S : rr.S_kept);
        }
      }
    }
    rr.px = px;
  }
  if (bad) rr.flags |= RF_BAD;
  __syncthreads();
  if (t == 0) {
    a.row[rl] = rr;
    a.pub[rl] = 0u;
  }
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
    sm.q.pidx[t] = a.kidx[(size_t)rlP * KEEP_CAP + t];
    sm.q.pprob[t] = a.kprob[(size_t)rlP * KEEP_CAP + t];
  }
  if (res && t < nq) {
    sm.q.qidx[t] = a.kidx[(size_t)rlQ * KEEP_CAP + t];
    sm.q.qprob[t] = a.kprob[(size_t)rlQ * KEEP_CAP + t];
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

template <int DT>
__device__ __forceinline__ double kept_prob(const char* rp, int j, const RowRec& R, bool filtered, double invT) {
  const float x = load_elem<DT>(rp, j);
  if (ord_key(x) < R.tau) return 0.0;
  return exp(((double)x - (double)R.m) * invT) / (filtered ? R.S_kept : R.S);
}

// Full-row draw by one workgroup (kept sets too large for a list; an empty
// residual of an unfiltered row).  Tiles of 2048 consecutive logits.
template <int DT>
__device__ int full_row_sample(const Args& a, double u, const char* pr, const RowRec& P, const char* qr,
                               const RowRec& Q, bool res, bool filtered, Smem& sm, double* Zout) {
  const int t = threadIdx.x, V = a.V;
  const double invT = a.invT;
  auto wt = [&](int j, bool use_res) -> double {
    const double p = kept_prob<DT>(pr, j, P, filtered, invT);
    if (!use_res) return p;
    const double d = p - kept_prob<DT>(qr, j, Q, filtered, invT);
    return d > 0.0 ? d : 0.0;
  };
  bool use_res = res;
  double Z = 0.0;
  int lastpos = -1;
  for (int pass = 0; pass < 2; ++pass) {
    Z = 0.0;
    lastpos = -1;
    for (int base = 0; base < V; base += SCE) {
      double ts = 0.0;
      for (int e = 0; e < 8; ++e) {
        const int j = base + t * 8 + e;
        if (j < V) {
          const double w = wt(j, use_res);
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
    double w8[8];
    double ts = 0.0;
    for (int e = 0; e < 8; ++e) {
      const int j = base + t * 8 + e;
      w8[e] = j < V ? wt(j, use_res) : 0.0;
      ts += w8[e];
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
      for (int e = 0; e < 8; ++e) {
        const int j = base + t * 8 + e;
        C += w8[e];
        if (j < V && w8[e] > 0.0) {
          lastp = j;
          if (first == INT_MAX && target < C) first = j;
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

template <int DT, int MODE>
__device__ void seq_finalize(const Args& a, int b, Smem& sm) {
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x, K = a.K, rps = a.rps;
  const RowRec* rr = a.row + (size_t)b * rps;
  __syncthreads();
  for (int j = t; j < rps; j += WG) {
    sm.q.px[j] = rr[j].px;
    sm.q.rf[j] = rr[j].flags;
  }
  __syncthreads();
  if (t == 0) {
    int bad = 0;
    for (int j = 0; j < rps; ++j) bad |= sm.q.rf[j] & RF_BAD;
    for (int i = 0; i < K; ++i) {
      const int x = a.X[(size_t)b * K + i];
      if (x < 0 || x >= a.V) bad = 1;
    }
    int n = K;
    for (int i = 0; i < K; ++i) {
      const double p = sm.q.px[i];
      bool acc;
      if (MODE == M_GREEDY) {
        acc = p > 0.0;
      } else {
        const double q = sm.q.px[K + 1 + i];
        acc = (double)a.U[(size_t)b * (K + 1) + i] * q < p;
      }
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
    for (int i = t; i < K; i += WG) {
      const double nanv = __longlong_as_double(0x7FF8000000000000ll);
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
    if (j < n) ot[j] = a.X[(size_t)b * K + j];
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
    tok = rr[n].arg;
  } else {
    const double u = (double)a.U[(size_t)b * (K + 1) + K];
    const bool res = n < K;
    const int rlP = b * rps + n, rlQ = b * rps + K + 1 + (res ? n : 0);
    const RowRec P = rr[n];
    const RowRec Q = rr[res ? K + 1 + n : n];
    if ((P.flags & RF_BIG) || (res && (Q.flags & RF_BIG))) {
      tok = full_row_sample<DT>(a, u, row_ptr(a, rlP, ESZ), P, row_ptr(a, res ? rlQ : rlP, ESZ), Q, res, true, sm,
                                &Z);
    } else {
      tok = list_sample(a, u, rlP, P.nkept, rlQ, res ? Q.nkept : 0, res, sm, &Z);
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

template <int DT, int MODE, bool VEC>
__global__ void __launch_bounds__(WG) stream_kernel(Args a) {
  __shared__ Smem sm;
  constexpr int ESZ = ElemT<DT>::ESZ;
  const int t = threadIdx.x;
  const int rl = (int)(blockIdx.x / (unsigned)a.nchunks);
  const int c = (int)blockIdx.x - rl * a.nchunks;
  const char* rp = row_ptr(a, rl, ESZ);
  const int c0 = c * CE, cn = min(CE, a.V - c0);

  float v[EPT];
  load_chunk<DT, VEC>(rp, c0, cn, v);
  float tm = -INFINITY;
#pragma unroll
  for (int k = 0; k < EPT; ++k) tm = fmaxf(tm, v[k]);
  const float mc = block_fmax(tm, sm.red);

  ChunkRec rec;
  rec.s = 0.0;
  rec.m = mc;
  rec.bound = 0u;
  rec.ncand = 0;
  rec.arg = 0;
  rec.pad0 = rec.pad1 = 0;

  if (MODE == M_PLAIN || MODE == M_TOPP) {
    float acc = 0.0f;
    if (mc > -INFINITY) {
      const float c2 = a.c2;
#pragma unroll
      for (int k = 0; k < EPT; ++k) acc += __builtin_amdgcn_exp2f((v[k] - mc) * c2);
    }
    rec.s = block_sum((double)acc, sm.red);
  }

  if (MODE == M_GREEDY) {
    int best = INT_MAX;
#pragma unroll
    for (int k = 0; k < EPT; ++k)
      if (v[k] == mc) best = min(best, local_index<DT, VEC>(k, t));
    best = block_min_i(best, sm.red);
    rec.arg = c0 + (best == INT_MAX ? 0 : best);
  }

  if (MODE == M_TOPP || MODE == M_TOPK || MODE == M_TOPKP) {
    uint32_t bound;
    if (MODE == M_TOPP) {
      // window below the larger of the chunk max and the row max published so far
      if (t == 0) sm.u0 = atomicMax(&a.pub[rl], ord_key(mc));
      __syncthreads();
      const float ref = sm.u0 > ord_key(mc) ? key_val(sm.u0) : mc;
      bound = ord_key(ref - a.win);
    } else {
      // k-th largest of the 256 thread maxima is <= the row's k-th largest logit
      sm.s.tk[t] = ord_key(tm);
      bitonic_desc(sm.s.tk, WG);
      // (for k > 256 no bound follows from 256 maxima: every finite logit qualifies)
      const uint32_t L = a.top_k <= WG ? (uint32_t)sm.s.tk[a.top_k - 1] : KEY_NEG_INF;
      if (t == 0) sm.u0 = atomicMax(&a.pub[rl], L);
      __syncthreads();
      bound = max(L, sm.u0);
    }
    // finite logits at or above the bound become candidates
    const float thr = bound > KEY_NEG_INF ? key_val(bound) : -3.402823466e38f;
    if (t == 0) sm.ncand = 0;
    __syncthreads();
    if (tm >= thr) {
#pragma unroll
      for (int k = 0; k < EPT; ++k) {
        if (v[k] >= thr) {
          const int s = atomicAdd(&sm.ncand, 1);
          if (s < CAND_CAP)
            sm.s.cand[s] = ((uint64_t)ord_key(v[k]) << 32) | (uint32_t)(c0 + local_index<DT, VEC>(k, t));
        }
      }
    }
    __syncthreads();
    const int nc = sm.ncand;
    uint64_t* dst = a.cand + (size_t)blockIdx.x * CAND_CAP;
    for (int s = t; s < min(nc, CAND_CAP); s += WG) dst[s] = sm.s.cand[s];
    rec.ncand = nc;
    rec.bound = bound;
  }
  if (t == 0) a.chunk[blockIdx.x] = rec;

  if (!last_arrival(&a.row_cnt[rl], (uint32_t)a.nchunks, &sm.flag)) return;
  row_finalize<DT, MODE>(a, rl, sm);
  if (!a.do_seq) return;
  const int b = rl / a.rps;
  if (!last_arrival(&a.seq_cnt[b], (uint32_t)a.rps, &sm.flag)) return;
  seq_finalize<DT, MODE>(a, b, sm);
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
      a.seg_sum[s] = ss;
      a.seg_last[s] = sl;
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
    loc += ssum[s];
    if (slast[s] >= 0) lastseg = s;
  }
  double Z;
  const double incl = block_incl_scan(loc, sm.red, &Z);
  lastseg = block_max_i(lastseg, sm.red);
  const double u = (double)a.U[(size_t)b * (K + 1) + K];
  int tok;
  if (!(Z > 0.0)) {
    // empty residual (round-off only): draw from p
    tok = full_row_sample<DT>(a, u, pr, P, qr, Q, false, false, sm, &Z);
  } else {
    const double target = u * Z;
    __syncthreads();
    sm.scan[t] = incl;
    __syncthreads();
    double run = t > 0 ? sm.scan[t - 1] : 0.0;
    int found = INT_MAX;
    double cstart = 0.0;
    for (int s = s0; s < s1; ++s) {
      const double ce = run + ssum[s];
      if (found == INT_MAX && target < ce) {
        found = s;
        cstart = run;
      }
      run = ce;
    }
    const int sf = block_min_i(found, sm.red);
    if (sf == INT_MAX) {
      tok = lastseg >= 0 ? slast[lastseg] : 0;
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
      tok = first != INT_MAX ? first : slast[sf];
      if (tok < 0) tok = lastseg >= 0 ? slast[lastseg] : 0;
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

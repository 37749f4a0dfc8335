// The output projection of a language model on the matrix cores: logits
// [M, V] (float32) = hidden [M, d] (bfloat16) x W^T, W [V, d] (bfloat16),
// both operands with d contiguous.  Each scored position's hidden state maps
// to one logit per vocabulary entry, and a decoding step spends its time
// reading W (page www.2kiu.com/news/5895634 §1; page www.cf-1.com/news/5155685
// §2.1); the target scores all K+1 positions of a round in one pass (page
// www.gsyq.cn/news/428210 §3.1), so W is read once for M = B(K+1) rows.
//
// Tiling (gfx950, v_mfma_f32_32x32x16_bf16, 64-wide waves):
//  * a workgroup (4 waves) owns a 128-row x 256-column tile of the output;
//    wave w owns columns [64w, 64w + 64) of it for all 128 rows: 4 x 2 blocks
//    of 32 x 32, 128 float32 accumulators per lane;
//  * both operands are staged in LDS in k blocks of 32 (128 hidden rows and
//    256 W rows of 64 bytes, rows padded to 80 bytes so that the fragment
//    reads of 16 consecutive rows fall in distinct banks), double-buffered
//    with one barrier per block; the global loads are whole 64-byte row
//    segments, four lanes per row, issued one block ahead;
//  * 61,440 bytes of LDS and at most 256 registers per lane keep two
//    workgroups (8 waves) on each compute unit, so one computes while the
//    other waits on its loads;
//  * lane half h of step s holds k = 16h + 8s + 0..7 of the block for both
//    operands (an order of the sum over k that both follow);
//  * the 128-row tiles of one 256-column W panel are consecutive tile ids
//    placed on one XCD (workgroup ids go round-robin over the 8 XCDs), so the
//    panel is read from HBM once and served to the other row tiles by that
//    XCD's L2;
//  * for the verification that follows, the epilogue can also reduce each
//    wave's 64 columns of every row to a tile record (max, and the tile's
//    exp2 sum or arg-max: TileStat), so that the chunk statistics need not
//    read the logits again (tile_stats).
#include "sv_common.hpp"

#include <atomic>
#include <cstddef>
#include <cstdint>

namespace sv {

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int LM_BM = 128;      // rows of hidden per tile
constexpr int LM_BN = 256;      // vocabulary entries per tile
constexpr int LM_BK = 32;       // k per staged block
constexpr int LM_WG = 256;      // threads (4 waves)
constexpr int LM_XCD = 8;       // XCDs the workgroup ids are dealt over
constexpr int LM_ROWB = 80;     // LDS bytes per staged row: 64 of data, 16 of padding

struct LmArgs {
  const uint16_t* H;  // [M, d] bfloat16 bit patterns
  const uint16_t* W;  // [V, d]
  float* C;           // [M, V]
  int32_t M, V, d;
  int32_t mtiles, ntiles, per_xcd;
  // tile statistics (stat != TS_NONE): records of rstride rows in R, this
  // projection's rows from row roff; c2 = log2(e) / T of its rows
  uint2* R;
  int32_t rstride, roff, stat;
  float c2;
};

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) { return __builtin_bit_cast(bf16x8, v); }

// Tile records of one wave's block of logits: rows row0 + 0 .. 32 mblocks - 1
// (those below M), columns col0 .. col0 + 63 (those below V; col0 is a
// multiple of TILE_N).  Lane (h, l32), accumulator r of block (mb, nb) holds
// row 32 mb + 8 (r / 4) + 4 h + r % 4, column col0 + 32 nb + l32.  Each
// 32-row block goes through the wave's own LDS tile (TS_LDS floats: 32 rows
// of 64 columns, rows padded to 68), and lane pair (2 rho, 2 rho + 1) then
// takes row rho, 32 columns a lane: the max, then the sum of exp2(x * c2 -
// Mt), Mt = ceil(max * c2) (every term at most 1; as the streaming kernel's
// sums against an integer offset), or the lowest column holding the max;
// the two lanes of a pair combine with one DPP swap (a + b on both, the
// same bits), and the even lane stores the record.
constexpr int TS_ROW = 68;
constexpr int TS_LDS = 32 * TS_ROW;
// lm_gemm_kernel: waves 0-1 take As, waves 2-3 Ws; lm_gemm_w8: 8 tiles in its staging LDS
static_assert(2 * TS_LDS * 4 <= 2 * LM_BM * LM_ROWB && 2 * TS_LDS * 4 <= 2 * LM_BN * LM_ROWB, "tile fits");
template <int MB>
__device__ __forceinline__ void tile_stats(const LmArgs& a, const f32x16 (&acc)[MB][2], float* lds, int row0,
                                           int mblocks, int col0, int h, int l32) {
  if (col0 >= a.V) return;
  const int lane = threadIdx.x & 63, rho = lane >> 1, eta = lane & 1;
  const int g = col0 / TILE_N;
  uint2* rg = a.R + ((size_t)(g / TILE_GROUP) * a.rstride + a.roff) * TILE_GROUP + g % TILE_GROUP;
  const int cb = col0 + 32 * eta;  // this lane's first column
  const int nval = min(32, a.V - cb);  // its columns below V (may be <= 0)
  const bool sum = a.stat == TS_SUM;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    if (mb >= mblocks) continue;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) lds[(8 * (r >> 2) + 4 * h + (r & 3)) * TS_ROW + 32 * nb + l32] = acc[mb][nb][r];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float x[32];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float4 v = *reinterpret_cast<const float4*>(lds + rho * TS_ROW + 32 * eta + 4 * k);
      x[4 * k] = v.x;
      x[4 * k + 1] = v.y;
      x[4 * k + 2] = v.z;
      x[4 * k + 3] = v.w;
    }
#pragma unroll
    for (int k = 0; k < 32; ++k) x[k] = k < nval ? x[k] : -INFINITY;
    uint32_t mk = ord_key(x[0]);
#pragma unroll
    for (int k = 1; k < 32; ++k) mk = max(mk, ord_key(x[k]));
    mk = max(mk, dpp_mov<DPP_QP_1032>(mk));
    const float m = key_val(mk);
    uint32_t v;
    if (sum) {
      const float Mt = fmaxf(__builtin_ceilf(m * a.c2), -1.0e30f);
      float e = 0.0f;
#pragma unroll
      for (int k = 0; k < 32; ++k) e += __builtin_amdgcn_exp2f(__builtin_fmaf(x[k], a.c2, -Mt));
      v = __float_as_uint(e + __uint_as_float(dpp_mov<DPP_QP_1032>(__float_as_uint(e))));
    } else {
      int c = INT_MAX;
#pragma unroll
      for (int k = 31; k >= 0; --k) c = x[k] == m ? cb + k : c;
      v = (uint32_t)min(c, (int)dpp_mov<DPP_QP_1032>((uint32_t)c));
    }
    const int row = row0 + 32 * mb + rho;
    if (eta == 0 && row < a.M) rg[(size_t)row * TILE_GROUP] = make_uint2(__float_as_uint(m), v);
  }
}

__global__ void __launch_bounds__(LM_WG, 2) lm_gemm_kernel(LmArgs a) {
  __shared__ __attribute__((aligned(16))) char As[2][LM_BM * LM_ROWB];
  __shared__ __attribute__((aligned(16))) char Ws[2][LM_BN * LM_ROWB];
  // tile q: consecutive ids within one XCD take consecutive tiles, and the
  // row tiles of a W panel are consecutive
  const int id = blockIdx.x;
  const int q = (id % LM_XCD) * a.per_xcd + id / LM_XCD;
  if (q >= a.mtiles * a.ntiles) return;
  const int nt = q / a.mtiles, mt = q - nt * a.mtiles;
  const int m0 = mt * LM_BM, n0 = nt * LM_BN;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int d = a.d, nkb = d / LM_BK;

  // staging role: thread t copies 16-byte chunk t % 4 of rows 64 i + t / 4
  // (hidden rows i < 2, W rows i < 4); rows past M or V read row 0 (a valid
  // address) and are zeroed in registers
  const int sr = t >> 2, sc = t & 3;
  const uint4* ap[2];
  const uint4* wp[4];
  bool aok[2], wok[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 64 * i + sr;
    aok[i] = m0 + r < a.M;
    ap[i] = reinterpret_cast<const uint4*>(a.H + (size_t)(aok[i] ? m0 + r : 0) * d) + sc;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 64 * i + sr;
    wok[i] = n0 + r < a.V;
    wp[i] = reinterpret_cast<const uint4*>(a.W + (size_t)(wok[i] ? n0 + r : 0) * d) + sc;
  }
  uint4 ra[2], rw[4];
  auto gload = [&](int kb) {
    const size_t o = (size_t)kb * (LM_BK / 8);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 v = ap[i][o];
      ra[i] = aok[i] ? v : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = wp[i][o];
      rw[i] = wok[i] ? v : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) *reinterpret_cast<uint4*>(As[buf] + (64 * i + sr) * LM_ROWB + 16 * sc) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(Ws[buf] + (64 * i + sr) * LM_ROWB + 16 * sc) = rw[i];
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;

  // a tile with at most 64 rows below M (the last one of M = 448, for one)
  // skips the matrix instructions of its empty lower half
  const bool full = a.M - m0 > 64;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const bool more = kb + 1 < nkb;
    if (more) gload(kb + 1);
    const int buf = kb & 1;
    const char* Ab = As[buf] + l32 * LM_ROWB + h * 32;
    const char* Bb = Ws[buf] + (64 * w + l32) * LM_ROWB + h * 32;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      bf16x8 bf[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bf[nb] = as_bf16x8(*reinterpret_cast<const uint4*>(Bb + nb * 32 * LM_ROWB + 16 * s));
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        if (mb < 2 || full) {
          const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(Ab + mb * 32 * LM_ROWB + 16 * s));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
    if (more) {
      lstore(buf ^ 1);
      __syncthreads();
    }
  }

  // lane (h, l32), accumulator r of 32 x 32 block (mb, nb) holds row
  // 32 mb + 8 (r / 4) + 4 h + r % 4, column 32 nb + l32 of the wave's columns
  const int mblocks = min(4, (a.M - m0 + 31) / 32);
  if (a.stat != TS_NONE) {
    // every wave is done with the staged operands: each takes TS_LDS floats of them
    __syncthreads();
    float* lds = w < 2 ? reinterpret_cast<float*>(As[0]) + w * TS_LDS : reinterpret_cast<float*>(Ws[0]) + (w - 2) * TS_LDS;
    tile_stats<4>(a, acc, lds, m0, mblocks, n0 + 64 * w, h, l32);
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = n0 + 64 * w + 32 * nb + l32;
    if (n >= a.V) continue;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      if (mb >= mblocks) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < a.M) __builtin_nontemporal_store(acc[mb][nb][r], a.C + (size_t)m * a.V + n);
      }
    }
  }
}

// The wide tiles: 64 MB rows x 256 columns per workgroup of 8 waves (2 x 4,
// each wave 32 MB x 64: MB = 4 as in lm_gemm_kernel, MB = 3 for row counts
// that fill 192-row tiles), k blocks of 64 (whole 128-byte lines of each
// operand row per load), both operands in LDS as 128-byte rows whose 16-byte
// chunks are XOR-swizzled by row (so the fragment reads of 16 consecutive
// rows hit distinct banks without padding), two stages: 128 KB (MB = 4) or
// 112 KB (MB = 3) of LDS, one workgroup per CU, fed from two register stages
// (each load is issued two k blocks before its block is multiplied).  Per
// flop the 256-row tile moves half the operand bytes of the 128-row tile
// from L2 and the 192-row tile three quarters (22% less); each W panel is
// staged by fewer workgroups.  The logits are written with non-temporal
// stores: only later launches read them.
__device__ __forceinline__ int sw64(int r, int c) { return r * 128 + 16 * (c ^ ((r >> 1) & 7)); }  // byte of chunk c, row r
template <int MB>
constexpr int w8_lds_bytes() { return 2 * (64 * MB + 256) * 128; }
template <int MB>
__global__ void __launch_bounds__(512, 1) lm_gemm_w8(LmArgs a) {
  constexpr int TM = 64 * MB;                        // rows of the tile
  constexpr int AST = TM * 128, WST = 256 * 128;     // bytes of one stage of each operand
  static_assert(8 * TS_LDS * 4 <= w8_lds_bytes<MB>(), "the epilogue's tiles fit the staging LDS");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* As = smem;                // [2][AST]
  char* Ws = smem + 2 * AST;      // [2][WST]
  const int id = blockIdx.x;
  const int q = (id % LM_XCD) * a.per_xcd + id / LM_XCD;
  if (q >= a.mtiles * a.ntiles) return;
  const int nt = q / a.mtiles, mt = q - nt * a.mtiles;
  const int m0 = mt * TM, n0 = nt * 256;
  const int t = threadIdx.x, lane = t & 63, w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const int d = a.d, nkb = d / 64;
  // staging role: 16-byte chunk t % 8 of rows 64 i + t / 8 (hidden rows i < MB,
  // W rows i < 4), read by buffer loads whose resource ends at the tile's
  // last row below M or V, so rows past them read as zeros
  const int sr = t >> 3, sc = t & 7;
  const char* abase = reinterpret_cast<const char*>(a.H + (size_t)m0 * d);
  const char* wbase = reinterpret_cast<const char*>(a.W + (size_t)n0 * d);
  const int abytes = min(TM, a.M - m0) * d * 2, wbytes = min(256, a.V - n0) * d * 2;
  int aoff[MB], woff[4];
#pragma unroll
  for (int i = 0; i < MB; ++i) aoff[i] = (64 * i + sr) * d * 2 + sc * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) woff[i] = (64 * i + sr) * d * 2 + sc * 16;
  // k block kb of both operands into registers: the resources start at the
  // block, so every offset stays below the bound exactly for valid rows
  auto gload = [&](uint4 (&ra)[MB], uint4 (&rw)[4], int kb) {
    const auto rsa = wave_rsrc(abase + kb * 128, abytes - kb * 128);
    const auto rsw = wave_rsrc(wbase + kb * 128, wbytes - kb * 128);
#pragma unroll
    for (int i = 0; i < MB; ++i) ra[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsa, aoff[i], 0, 0));
#pragma unroll
    for (int i = 0; i < 4; ++i) rw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsw, woff[i], 0, 0));
  };
  auto lstore = [&](const uint4 (&ra)[MB], const uint4 (&rw)[4], int buf) {
#pragma unroll
    for (int i = 0; i < MB; ++i) *reinterpret_cast<uint4*>(As + buf * AST + sw64(64 * i + sr, sc)) = ra[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(Ws + buf * WST + sw64(64 * i + sr, sc)) = rw[i];
  };
  f32x16 acc[MB][2];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nb][r] = 0.0f;
  // this wave's first row; the wave skips the matrix instructions of its
  // 32-row blocks that lie wholly past M
  const int wrow0 = m0 + 32 * MB * wm;
  const int nblk = a.M > wrow0 ? min(MB, (a.M - wrow0 + 31) / 32) : 0;
  auto compute = [&](int buf) {
    const char* Ab = As + buf * AST;
    const char* Bb = Ws + buf * WST;
    if (nblk == 0) return;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // lane half h of step s holds chunk c: k = 8c .. 8c + 7 of the block
      const int c = 2 * h + (s & 1) + 4 * (s >> 1);
      bf16x8 bf[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) bf[nb] = as_bf16x8(*reinterpret_cast<const uint4*>(Bb + sw64(64 * wn + 32 * nb + l32, c)));
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        if (mb < nblk) {
          const bf16x8 af = as_bf16x8(*reinterpret_cast<const uint4*>(Ab + sw64(32 * MB * wm + 32 * mb + l32, c)));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
  };
  // Two register stages ahead of the LDS stage.  Pass b first stores block
  // b + 1 from its register set into the LDS stage that block b - 1 used
  // (free since the last barrier), refills that set with block b + 3, then
  // multiplies block b from LDS; one barrier ends the pass.  Each load thus
  // has two blocks of matrix work to arrive in, and the stores overlap the
  // other waves' matrix work instead of sitting before the barrier (3-4%
  // faster than storing after the multiply).  The loop runs two blocks per
  // iteration so that the register sets are named statically; past the last
  // block the loads repeat it (in bounds, unused).
  uint4 ra0[MB], rw0[4], ra1[MB], rw1[4];
  gload(ra0, rw0, 0);
  gload(ra1, rw1, min(1, nkb - 1));
  lstore(ra0, rw0, 0);
  gload(ra0, rw0, min(2, nkb - 1));
  __syncthreads();
  // set 1 holds block 1 and set 0 block 2
  for (int kb = 0; kb < nkb; kb += 2) {
    if (kb + 1 < nkb) lstore(ra1, rw1, 1);
    gload(ra1, rw1, min(kb + 3, nkb - 1));
    compute(0);
    __syncthreads();
    if (kb + 1 >= nkb) break;
    if (kb + 2 < nkb) lstore(ra0, rw0, 0);
    gload(ra0, rw0, min(kb + 4, nkb - 1));
    compute(1);
    __syncthreads();
  }
  if (a.stat != TS_NONE) {
    // every wave is done with the staged operands: each takes TS_LDS floats of them
    __syncthreads();
    tile_stats<MB>(a, acc, reinterpret_cast<float*>(smem) + w * TS_LDS, wrow0, nblk, n0 + 64 * wn, h, l32);
  }
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int n = n0 + 64 * wn + 32 * nb + l32;
    if (n >= a.V) continue;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      if (mb >= nblk) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = wrow0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < a.M) __builtin_nontemporal_store(acc[mb][nb][r], a.C + (size_t)m * a.V + n);
      }
    }
  }
}

}  // namespace

// Shapes the caller has checked: M >= 1, V >= 1, d a positive multiple of 64 (k blocks of 32 and 64),
// H, W 16-byte aligned, the tile count within the grid limit.  With stat !=
// TS_NONE the epilogue also writes the tile records of the M rows to R, as
// rows roff .. roff + M - 1 of rstride (records of 64-column tiles, grouped by
// 256 columns: TileStat), with c2 = log2(e) / T.
namespace {

// Launches the wide-tile kernel of 64 MB-row tiles; its dynamic LDS limit is
// raised once per device (setting it twice from racing first calls is harmless).
template <int MB>
hipError_t launch_w8(LmArgs a, hipStream_t s) {
  constexpr int TM = 64 * MB;
  a.mtiles = (a.M + TM - 1) / TM;
  a.ntiles = (a.V + 255) / 256;
  a.per_xcd = (a.mtiles * a.ntiles + LM_XCD - 1) / LM_XCD;
  static std::atomic<bool> attr_set[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  if (!attr_set[dev].load(std::memory_order_acquire)) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)lm_gemm_w8<MB>, hipFuncAttributeMaxDynamicSharedMemorySize, w8_lds_bytes<MB>());
    if (e != hipSuccess) return e;
    attr_set[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL(lm_gemm_w8<MB>, dim3((unsigned)(a.per_xcd * LM_XCD)), dim3(512), w8_lds_bytes<MB>(), s, a);
  return hipGetLastError();
}

// Rows wasted in the last tile of M rows, as a fraction of the tiles' rows.
double tile_waste(int32_t M, int tm) { return 1.0 - (double)M / ((double)tm * ((M + tm - 1) / tm)); }

}  // namespace

hipError_t launch_lm_gemm(const void* H, const void* W, float* C, int32_t M, int32_t V, int32_t d, hipStream_t s,
                          void* R, int32_t rstride, int32_t roff, int stat, float c2) {
  LmArgs a;
  a.H = static_cast<const uint16_t*>(H);
  a.W = static_cast<const uint16_t*>(W);
  a.C = C;
  a.M = M;
  a.V = V;
  a.d = d;
  a.R = static_cast<uint2*>(R);
  a.rstride = rstride;
  a.roff = roff;
  a.stat = R ? stat : TS_NONE;
  a.c2 = c2;
  // The larger tile when its row tiles waste no more rows than the 128-row
  // tile's (plus 5%): M = 448 takes 256-row tiles, M = 384 192-row tiles.
  const double w128 = tile_waste(M, 128), w192 = tile_waste(M, 192), w256 = tile_waste(M, 256);
  if (d % 64 == 0 && w256 <= w128 + 0.05 && w256 <= w192) return launch_w8<4>(a, s);
  if (d % 64 == 0 && w192 <= w128 + 0.05) return launch_w8<3>(a, s);
  a.mtiles = (M + LM_BM - 1) / LM_BM;
  a.ntiles = (V + LM_BN - 1) / LM_BN;
  a.per_xcd = (a.mtiles * a.ntiles + LM_XCD - 1) / LM_XCD;
  hipLaunchKernelGGL(lm_gemm_kernel, dim3((unsigned)(a.per_xcd * LM_XCD)), dim3(LM_WG), 0, s, a);
  return hipGetLastError();
}

int64_t lm_gemm_tiles(int32_t M, int32_t V) {
  return (int64_t)((M + LM_BM - 1) / LM_BM) * ((V + LM_BN - 1) / LM_BN);
}

}  // namespace sv

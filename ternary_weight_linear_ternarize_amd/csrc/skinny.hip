// Few tokens (M <= 16): weights straight from HBM into MFMA operand registers.
//
// Same operands as the other product kernels -- int8 activations [M][Kp],
// packed 2-bit weights, acc = sum q (t + 1) - rowsum.  Each wave owns one
// 16-row weight tile over a range of 256-weight blocks (KS waves share a
// tile's K when the layer has too few rows to fill the GPU).  Lane (g, li)
// loads the 16 bytes it feeds to the MFMA itself -- words 4g .. 4g+3 of
// block b of weight row li, i.e. 64 contiguous bytes per row and load -- so
// nothing is staged in LDS on the weight side: every weight load of a wave
// is issued up front and each block waits only for its own data (vmcnt
// counts in order).  Measured on this chip, 64-byte row pieces stream at
// about 5 TB/s, against about 5.9 TB/s for 128 bytes and more; the LDS
// write and read-back that a row-contiguous load needs cost more than that.
// The activations (M rows) are staged once per block through registers;
// lanes of token rows >= M skip their operand reads (exec-masked: the LDS
// does no work for them), which halves the activation traffic at 8 tokens.
//
// k-step s of block b: lane (g, li) feeds activation bytes 256 b + 64 g +
// 16 s .. +15 of token row li and word 4g + s of weight row li.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

enum { SK_DSTORE = 0, SK_DGATEUP = 1 };

// NBLK: 256-weight blocks per wave (upper bound); XR: 16-byte activation
// pieces per thread; WPB waves per block.  KS (waves per tile) divides WPB.
template <int NB, int NBLK, int XR, int WPB, int EPI>
__global__ __launch_bounds__(64 * WPB) void mfma_direct_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int M, int64_t Kp, const uint32_t* __restrict__ W0,
    const float* __restrict__ s0, const uint32_t* __restrict__ W1, const float* __restrict__ s1,
    int64_t N, float* __restrict__ Y, int32_t* __restrict__ acc_out, float* __restrict__ gh_parts,
    int KS) {
  constexpr int NT = 64 * WPB;
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  __shared__ float red[WPB][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int tpb = WPB / KS;
  const int tile = wave / KS, kpart = wave % KS;
  const int pitch = (int)Kp + 16;
  int8_t* lds_x = lds;
  // partial accumulators of the K split, after the staged rows (+256 B: the
  // operand reads of a partial last block run past Kp)
  v4i* lds_part = reinterpret_cast<v4i*>(lds + ((M * pitch + 15) / 16) * 16 + 256);
  const int nblk = (int)((Kp + 255) / 256);
  const int b0 = kpart * nblk / KS, b1 = (kpart + 1) * nblk / KS;  // this wave's blocks
  const int64_t wpr = Kp / 16;
  const int64_t nbase = (int64_t)blockIdx.x * (16 * tpb) + 16 * tile;
  int64_t nrow = nbase + li;
  nrow = nrow < N ? nrow : N - 1;

  // activation pieces first: staged row r, piece col < ppr holds codes for col < kpp
  const int ppr = pitch / 16, kpp = (int)(Kp / 16), total = M * ppr;
  // (buffer loads: the compiler keeps them where they are written, ahead of
  // the weight loads, so the staging below waits only for them; a plain load
  // sunk to its store after the weight loads would wait for everything)
  TokenOperands<1> tok;  // the epilogue's scales and row sums, before everything else
  tok.load(x_scale, rowsum, M, 0);
  const float ws0 = s0[0], ws1 = NB == 2 ? s1[0] : 0.0f;  // weight scales, also early
  const buf_rsrc rx = make_buf_rsrc(Xq, (uint32_t)(M * Kp));
  u32x4 xr[XR];
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    int pc = tid + NT * j;
    pc = pc < total ? pc : total - 1;
    const int row = pc / ppr;
    int col = pc - row * ppr;
    col = col < kpp ? col : kpp - 1;
    xr[j] = __builtin_amdgcn_raw_buffer_load_b128(rx, (uint32_t)(row * Kp + 16 * col), 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  // every weight load of the wave: buffer loads at one offset register plus
  // immediates (past the matrix they read zero; words past a row's end are
  // zeroed where they are used)
  u32x4 wv[NB][NBLK];
  const uint32_t voff = (uint32_t)((nrow * wpr + 16 * (int64_t)b0 + 4 * g) * 4);
#pragma unroll
  for (int mat = 0; mat < NB; ++mat) {
    const buf_rsrc rw = make_buf_rsrc(mat == 0 ? W0 : W1, (uint32_t)(N * wpr * 4));
#pragma unroll
    for (int b = 0; b < NBLK; ++b)
      wv[mat][b] = __builtin_amdgcn_raw_buffer_load_b128(rw, voff + 64 * b, 0, 2);  // nt
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads issued before the staging waits
  // straight-line stores of every loaded piece (threads past the end rewrite
  // the last piece; the pad piece of a row gets a copy of its last one: it
  // only meets zero weights)
#pragma unroll
  for (int j = 0; j < XR; ++j) {
    int pc = tid + NT * j;
    pc = pc < total ? pc : total - 1;
    const int row = pc / ppr, col = pc - row * ppr;
    *reinterpret_cast<u32x4*>(lds_x + row * pitch + 16 * col) = xr[j];
  }
  __syncthreads();

  v4i acc[NB][2];
#pragma unroll
  for (int mat = 0; mat < NB; ++mat) acc[mat][0] = acc[mat][1] = v4i{0, 0, 0, 0};
  const bool arow = li < M;
  const int8_t* xrow = lds_x + (arow ? li : 0) * pitch + 64 * g;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    if (b0 + b < b1) {
      const int blk = b0 + b;
      const bool wok = 16 * (int64_t)blk + 4 * g < wpr;  // past Kp: zero codes
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        v4i av = v4i{0, 0, 0, 0};
        if (arow) av = *reinterpret_cast<const v4i*>(xrow + 256 * blk + 16 * s);
#pragma unroll
        for (int mat = 0; mat < NB; ++mat) {
          uint32_t wd = wv[mat][b][s];
          wd = wok ? wd : 0u;
          acc[mat][s & 1] =
              __builtin_amdgcn_mfma_i32_16x16x64_i8(av, codes_operand(wd), acc[mat][s & 1], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int mat = 0; mat < NB; ++mat) acc[mat][0] += acc[mat][1];

  // K split: waves 1 .. KS-1 of a tile hand their partial sums to wave 0
  if (KS > 1) {
    if (kpart > 0) {
#pragma unroll
      for (int mat = 0; mat < NB; ++mat)
        lds_part[((tile * (KS - 1) + kpart - 1) * NB + mat) * 64 + lane] = acc[mat][0];
    }
    __syncthreads();
    if (kpart == 0) {
      for (int k = 1; k < KS; ++k)
#pragma unroll
        for (int mat = 0; mat < NB; ++mat)
          acc[mat][0] += lds_part[((tile * (KS - 1) + k - 1) * NB + mat) * 64 + lane];
    }
  }
  const bool owner = kpart == 0;

  // result lane l, register r: token 4g + r, weight row nbase + li
  const int64_t n = nbase + li;
  if constexpr (EPI == SK_DSTORE) {
    const float sw = ws0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (owner && m < M && n < N) {
        const int a = acc[0][0][r] - tok.rs[0][r];
        if (Y) Y[(int64_t)m * N + n] = dequant_fast(a, __fmul_rn(sw, tok.xs[0][r]));
        if (acc_out) acc_out[(int64_t)m * N + n] = a;
      }
    }
  } else {
    const float sg = ws0, su = ws1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      float hm = 0.0f;
      if (owner && m < M && n < N) {
        const int32_t rsm = tok.rs[0][r];
        const float xs = tok.xs[0][r];
        const float gv = dequant_fast(acc[0][0][r] - rsm, __fmul_rn(sg, xs));
        const float uv = dequant_fast(acc[NB - 1][0][r] - rsm, __fmul_rn(su, xs));
        const float t = gv > 0.0f ? gv : 0.0f;
        const float h = __fmul_rn(__fmul_rn(t, t), uv);
        Y[(int64_t)m * N + n] = h;
        hm = fabsf(h);
      }
      // max over the 16 lanes holding this token row (lane bits 0..3)
      hm = fmaxf(hm, __int_as_float(dpp::xchg<8>(__float_as_int(hm))));
      hm = fmaxf(hm, __int_as_float(dpp::xchg<4>(__float_as_int(hm))));
      hm = fmaxf(hm, __int_as_float(dpp::xchg<2>(__float_as_int(hm))));
      hm = fmaxf(hm, __int_as_float(dpp::xchg<1>(__float_as_int(hm))));
      if (li == 0) red[wave][m] = hm;
    }
    __syncthreads();
    if (tid < M) {
      float v = 0.0f;
      for (int w = 0; w < WPB; w += KS) v = fmaxf(v, red[w][tid]);
      gh_parts[(int64_t)blockIdx.x * M + tid] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side.

static int64_t dir_lds(int64_t M, int64_t Kp, int nb, int wpb, int ks) {
  return ((M * (Kp + 16) + 15) / 16) * 16 + 256 + (int64_t)(wpb / ks) * (ks - 1) * nb * 1024;
}

constexpr int64_t kDirLds = 144 * 1024;

struct DirPlan {
  int ks, wpb, nblk_b, xr_b;  // waves per tile and block, 256-weight blocks, pieces buckets
  bool ok;
};

// Waves per tile: enough waves (about 1500) for the 256 CUs, registers for
// the wave's weights bounded (NB x blocks <= 32 uint4, 16 for M > 8 whose
// activation pieces take more registers).  Four waves per block unless the
// K split needs eight (more blocks, each CU holding two).
static DirPlan dir_plan(int64_t M, int64_t Kp, int64_t N, int nb) {
  DirPlan p{};
  const int64_t tiles = (N + 15) / 16, nblk = (Kp + 255) / 256;
  const int64_t cap = M > 8 ? 16 : 32;
  int ks = 1;
  while (ks < 8 && (tiles * ks < 1500 || nb * ((nblk + ks - 1) / ks) > cap)) ks *= 2;
  const int64_t per = (nblk + ks - 1) / ks;
  p.ks = ks;
  p.wpb = ks <= 4 ? 4 : 8;
  p.nblk_b = per <= 4 ? 4 : per <= 8 ? 8 : per <= 16 ? 16 : 32;
  const int64_t xr = (M * ((Kp + 16) / 16) + 64 * p.wpb - 1) / (64 * p.wpb);
  p.xr_b = xr <= 3 ? 3 : xr <= 9 ? 9 : xr <= 17 ? 17 : 33;
  // Only for layers whose K is split over several waves (the FFN's shapes):
  // with the whole K in one wave (the 100B-class layer) the streaming kernel
  // of gemm.hip measured faster (17.6 against 21.6 us at 8 tokens), this
  // kernel's per-wave compute (about 13 us with the weight loads removed)
  // not hiding under its memory time.
  p.ok = ks >= 2 && M >= 1 && M <= 16 && nb * p.nblk_b <= 32 && per <= 32 && xr <= 33 &&
         nb * p.nblk_b + p.xr_b <= (p.wpb == 4 ? 52 : 48) &&  // registers (uint4): no spills
         dir_lds(M, Kp, nb, p.wpb, ks) <= kDirLds;
  return p;
}

template <int NB, int NBLK, int XR, int WPB, int EPI>
static hipError_t dir_go(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                         int64_t Kp, const uint32_t* W0, const float* s0, const uint32_t* W1,
                         const float* s1, int64_t N, float* Y, int32_t* acc_out, float* gh_parts,
                         int* nparts, const DirPlan& p, hipStream_t s) {
  auto kern = mfma_direct_kernel<NB, NBLK, XR, WPB, EPI>;
  static bool once = ((void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                (int)kDirLds),
                      true);
  (void)once;
  const int tpb = WPB / p.ks;
  const unsigned blocks = (unsigned)((N + 16 * tpb - 1) / (16 * tpb));
  if (nparts) *nparts = (int)blocks;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(64 * WPB), (size_t)dir_lds(M, Kp, NB, WPB, p.ks),
                     s, Xq, xs, rs, (int)M, Kp, W0, s0, W1, s1, N, Y, acc_out, gh_parts, p.ks);
  return hipGetLastError();
}

template <int NB, int EPI>
static hipError_t dir_dispatch(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                               int64_t Kp, const uint32_t* W0, const float* s0, const uint32_t* W1,
                               const float* s1, int64_t N, float* Y, int32_t* acc_out,
                               float* gh_parts, int* nparts, const DirPlan& p, hipStream_t s) {
#define BL_DIR(NBLK, XR, WPB)                                                                   \
  return dir_go<NB, NBLK, XR, WPB, EPI>(Xq, xs, rs, M, Kp, W0, s0, W1, s1, N, Y, acc_out,     \
                                        gh_parts, nparts, p, s)
#define BL_DIR_W(NBLK, XR)                          \
  if (p.wpb == 4) BL_DIR(NBLK, XR, 4); \
  BL_DIR(NBLK, XR, 8)
#define BL_DIR_XR(NBLK)                        \
  if (p.xr_b == 3) { BL_DIR_W(NBLK, 3); }      \
  if (p.xr_b == 9) { BL_DIR_W(NBLK, 9); }      \
  if (p.xr_b == 17) { BL_DIR_W(NBLK, 17); }    \
  BL_DIR_W(NBLK, 33)
  if (p.nblk_b == 4) { BL_DIR_XR(4); }
  if (p.nblk_b == 8) { BL_DIR_XR(8); }
  if constexpr (NB == 1) {
    if (p.nblk_b == 16) { BL_DIR_XR(16); }
    BL_DIR_XR(32);
  } else {
    BL_DIR_XR(16);
  }
#undef BL_DIR_XR
#undef BL_DIR_W
#undef BL_DIR
}

bool direct_ok(int64_t M, int64_t K, int64_t N, int nb) {
  return dir_plan(M, (K + 63) / 64 * 64, N, nb).ok;
}

hipError_t launch_direct(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                         int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                         int32_t* acc_out, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  const DirPlan p = dir_plan(M, Kp, N, 1);
  if (!p.ok) return hipErrorInvalidValue;
  return dir_dispatch<1, SK_DSTORE>(Xq, xs, rs, M, Kp, Wp, ws, nullptr, nullptr, N, Y, acc_out,
                                    nullptr, nullptr, p, s);
}

hipError_t launch_direct_gateup(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                                int64_t K, const uint32_t* Wg, const float* sg,
                                const uint32_t* Wu, const float* su, int64_t N, float* H,
                                float* gh_parts, int* nparts, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  const DirPlan p = dir_plan(M, Kp, N, 2);
  if (!p.ok) return hipErrorInvalidValue;
  return dir_dispatch<2, SK_DGATEUP>(Xq, xs, rs, M, Kp, Wg, sg, Wu, su, N, H, nullptr, gh_parts,
                                     nparts, p, s);
}

}  // namespace bl

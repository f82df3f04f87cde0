// Split-K skinny GEMM for up to 64 tokens (the FFN's down projection).
//
// Same operands as the other product kernels -- activations int8 [M][Kp],
// packed 2-bit weights, acc = sum q (t + 1) - rowsum -- for layers with few
// weight rows, where one tile per wave over the whole K leaves too few waves
// in flight (the FFN's down projection has 2560 rows, 160 tiles of 16).  The
// grid is (weight-row blocks) x (K parts): each block stages its K part of
// the activations (M rows) in LDS once, with every load in flight, and each
// of its waves streams one 16-row weight tile over that K part the way
// mfma_stream_kernel does (row-contiguous 16-byte lanes into a wave-private
// LDS patch, then v_mfma_i32_16x16x64_i8 with M/16 token tiles sharing each
// unpacked weight operand).  With one K part the kernel runs the epilogue
// itself; otherwise the int32 partial sums go to a workspace and
// splitk_reduce_kernel adds the K parts (integer adds: the order does not
// matter) and dequantises.  A last-arriving-block reduction inside the first
// kernel was measured an order of magnitude slower on this chip: its
// device-scope release fences cost far more than a second launch.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

template <int TMS, int LPR, int WPB>
__global__ __launch_bounds__(64 * WPB) void mfma_splitk_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int M, int64_t Kp, const uint32_t* __restrict__ W,
    const float* __restrict__ w_scale, int64_t N, float* __restrict__ Y,
    int32_t* __restrict__ part, int ksb) {
  constexpr int STEP = LPR * 64;     // weights per row per step (16 B per lane)
  constexpr int RPI = 64 / LPR;      // rows per load instruction
  constexpr int NI = 16 / RPI;       // load instructions per matrix per step
  constexpr int BP = STEP / 4 + 16;  // bytes per staged weight row (+ pad)
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  const int kb = blockIdx.x % ksb, tb = blockIdx.x / ksb;
  const int nsteps_all = (int)((Kp + STEP - 1) / STEP);
  const int sb = kb * nsteps_all / ksb, se = (kb + 1) * nsteps_all / ksb;
  const int nsteps = se - sb;
  const int64_t kbeg = (int64_t)sb * STEP;
  const int64_t kend = (int64_t)se * STEP < Kp ? (int64_t)se * STEP : Kp;
  const int64_t klen = kend - kbeg;  // a multiple of 64
  const int64_t pitch = klen + 16;   // staged activation row (+16 B spreads the banks)
  int8_t* lds_x = lds;
  int8_t* lds_w = lds + staged_rows_bytes(M, pitch) + (int64_t)wave * 16 * BP;
  const int64_t wpr = Kp / 16;
  const int C = (int)(Kp / 64);
  const int64_t nbase = (int64_t)tb * (16 * WPB) + 16 * wave;
  const int lr = lane / LPR, lc = lane % LPR;

  uint4 st[NI];
  auto load_step = [&](int sidx) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int64_t n = nbase + RPI * i + lr;
      n = n < N ? n : N - 1;
      const int c = (sb + sidx) * LPR + lc;
      st[i] = c < C ? load_stream_u4(reinterpret_cast<const uint4*>(W + n * wpr) + c)
                    : make_uint4(0x55555555u, 0x55555555u, 0x55555555u, 0x55555555u);
    }
  };
  auto stage_step = [&]() {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<uint4*>(lds_w + (RPI * i + lr) * BP + 16 * lc) = st[i];
  };
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if (nsteps > 0) load_step(0);
  // this block's K part of the activations -> LDS, every load in flight at once
  stage_rows_lds<64 * WPB>(Xq, Kp, M, kbeg, (int)klen, (int)pitch, lds_x);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  v4i acc[TMS][2];
#pragma unroll
  for (int tm = 0; tm < TMS; ++tm) acc[tm][0] = acc[tm][1] = v4i{0, 0, 0, 0};

  for (int sidx = 0; sidx < nsteps; ++sidx) {
    stage_step();
    wave_sync();
    if (sidx + 1 < nsteps) load_step(sidx + 1);
    const int64_t k0 = (int64_t)sidx * STEP;  // relative to kbeg
#pragma unroll
    for (int b = 0; b < STEP / 256; ++b) {
      if (k0 + 256 * b < klen) {
        const uint4 bw = *reinterpret_cast<const uint4*>(lds_w + li * BP + 64 * b + 16 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          // lane (g, li): activation bytes 64 g + 16 s of the 256-weight block,
          // packed word 4 g + s of its weight row
          const int64_t ka = k0 + 256 * b + 64 * g + 16 * s;
          const uint32_t wd = s == 0 ? bw.x : s == 1 ? bw.y : s == 2 ? bw.z : bw.w;
          const v4i bv = codes_operand(wd);
#pragma unroll
          for (int tm = 0; tm < TMS; ++tm) {
            const int row = 16 * tm + li;
            // past klen (a tail 256-block) the staged row ends: zero operand
            const v4i a = (row < M && ka < klen)
                              ? *reinterpret_cast<const v4i*>(lds_x + row * pitch + ka)
                              : v4i{0, 0, 0, 0};
            acc[tm][s & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bv, acc[tm][s & 1], 0, 0, 0);
          }
        }
      }
    }
    wave_sync();
  }
#pragma unroll
  for (int tm = 0; tm < TMS; ++tm) acc[tm][0] += acc[tm][1];

  // result lane l, register r of token tile tm: token 16 tm + 4 g + r, weight row nbase + li
  const int64_t n = nbase + li;
  if (ksb > 1) {  // partial sums; splitk_reduce_kernel finishes
    int32_t* dst = part + (int64_t)kb * M * N;
#pragma unroll
    for (int tm = 0; tm < TMS; ++tm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * tm + 4 * g + r;
        if (m < M && n < N) dst[(int64_t)m * N + n] = acc[tm][0][r];
      }
    return;
  }
  const float sw = w_scale[0];
#pragma unroll
  for (int tm = 0; tm < TMS; ++tm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * tm + 4 * g + r;
      if (m < M && n < N)
        Y[(int64_t)m * N + n] = dequant_fast(acc[tm][0][r] - rowsum[m], __fmul_rn(sw, x_scale[m]));
    }
}

// Adds the K parts of the partial sums and dequantises.  Thread t of block
// (m, nb) covers token row m, columns 4 (256 nb + t) .. +3 (N % 4 == 0).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(
    const int32_t* __restrict__ part, int ksb, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int64_t M, int64_t N, const float* __restrict__ w_scale,
    float* __restrict__ Y, int nnb) {
  const int64_t m = blockIdx.x / nnb;
  const int nb = blockIdx.x % nnb;
  const int64_t n = 4 * ((int64_t)nb * 256 + threadIdx.x);
  if (n >= N) return;
  const int64_t plane = M * N;
  int4 a = make_int4(0, 0, 0, 0);
  for (int k = 0; k < ksb; ++k) {
    const int4 v = *reinterpret_cast<const int4*>(part + k * plane + m * N + n);
    a.x += v.x;
    a.y += v.y;
    a.z += v.z;
    a.w += v.w;
  }
  const int32_t rsm = rowsum[m];
  const float sc = __fmul_rn(w_scale[0], x_scale[m]);
  float4 y;
  y.x = dequant_fast(a.x - rsm, sc);
  y.y = dequant_fast(a.y - rsm, sc);
  y.z = dequant_fast(a.z - rsm, sc);
  y.w = dequant_fast(a.w - rsm, sc);
  *reinterpret_cast<float4*>(Y + m * N + n) = y;
}

// ---------------------------------------------------------------------------
// Host side.

constexpr int kSplitLpr = 8;                 // STEP = 512 weights
constexpr int kSplitWpb = 4;                 // 16-row tiles per block
constexpr int kSplitBp = kSplitLpr * 16 + 16;
constexpr int64_t kSplitLds = 144 * 1024;    // hard limit (dynamic LDS allowed)
constexpr int64_t kSplitLdsTwo = 76 * 1024;  // two blocks per CU

static int64_t splitk_lds(int64_t M, int64_t klen) {
  return staged_rows_bytes(M, klen + 16) + (int64_t)kSplitWpb * 16 * kSplitBp;
}

SplitPlan splitk_plan(int64_t M, int64_t K, int64_t N) {
  SplitPlan p{};
  const int64_t Kp = (K + 63) / 64 * 64;
  const int64_t step = 64 * kSplitLpr;
  const int64_t nsteps = (Kp + step - 1) / step;
  p.ntb = (N + 16 * kSplitWpb - 1) / (16 * kSplitWpb);
  // enough blocks for the 256 CUs (about 320), each K part small enough for
  // two blocks per CU where possible
  int64_t ksb = (320 + p.ntb - 1) / p.ntb;
  if (ksb > nsteps) ksb = nsteps;
  if (ksb < 1) ksb = 1;
  while (ksb < nsteps && splitk_lds(M, ((nsteps + ksb - 1) / ksb) * step) > kSplitLdsTwo) ++ksb;
  p.ksb = ksb;
  p.part_elems = ksb > 1 ? ksb * M * N : 0;
  p.ok = M >= 1 && M <= 64 && N % 4 == 0 &&
         splitk_lds(M, ((nsteps + ksb - 1) / ksb) * step) <= kSplitLds;
  return p;
}

template <int TMS>
static hipError_t splitk_go(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                            int64_t Kp, const uint32_t* W, const float* ws, int64_t N, float* Y,
                            int32_t* part, const SplitPlan& p, hipStream_t s) {
  auto kern = mfma_splitk_kernel<TMS, kSplitLpr, kSplitWpb>;
  static bool once = ((void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                (int)kSplitLds),
                      true);
  (void)once;
  const int64_t step = 64 * kSplitLpr;
  const int64_t nsteps = (Kp + step - 1) / step;
  int64_t lds = 0;  // the largest K part
  for (int64_t kb = 0; kb < p.ksb; ++kb) {
    const int64_t sb = kb * nsteps / p.ksb, se = (kb + 1) * nsteps / p.ksb;
    const int64_t klen = (se * step < Kp ? se * step : Kp) - sb * step;
    lds = lds > splitk_lds(M, klen) ? lds : splitk_lds(M, klen);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(p.ntb * p.ksb)), dim3(64 * kSplitWpb), (size_t)lds, s,
                     Xq, xs, rs, (int)M, Kp, W, ws, N, Y, part, (int)p.ksb);
  if (p.ksb > 1) {
    const int nnb = (int)((N / 4 + 255) / 256);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)(M * nnb)), dim3(256), 0, s, part,
                       (int)p.ksb, xs, rs, M, N, ws, Y, nnb);
  }
  return hipGetLastError();
}

hipError_t launch_splitk(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                         int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                         int32_t* part, hipStream_t s) {
  const SplitPlan p = splitk_plan(M, K, N);
  if (!p.ok) return hipErrorInvalidValue;
  const int64_t Kp = (K + 63) / 64 * 64;
  if (M <= 16) return splitk_go<1>(Xq, xs, rs, M, Kp, Wp, ws, N, Y, part, p, s);
  if (M <= 32) return splitk_go<2>(Xq, xs, rs, M, Kp, Wp, ws, N, Y, part, p, s);
  if (M <= 48) return splitk_go<3>(Xq, xs, rs, M, Kp, Wp, ws, N, Y, part, p, s);
  return splitk_go<4>(Xq, xs, rs, M, Kp, Wp, ws, N, Y, part, p, s);
}

}  // namespace bl

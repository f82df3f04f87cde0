// Binary weights in the 1-bit layout (youngju.dev "BitNet論文分析", section
// "1-Bit重みとSign関数": W_b = Sign(W), two values, so one bit per weight).
//
// Row n of Wb holds Kb = K rounded up to 128 weights as Kb/32 words; weight
// 32j + 4s + b is bit 8b + s of word j (1 = +1, 0 = -1; padding bits 0).
// Half the bytes of the 2-bit codes, which for binary weights only ever hold
// 00 and 10: the 1-bit layout drops the always-zero low bit.
//
// The product is taken as acc = sum_k q (t + 1) - rowsum with t + 1 = 2 bit,
// the same shifted-code form as the 2-bit kernels:
//  * one token: gemv1_kernel, the GEMV of gemv.hip with 128 weights (one
//    16-byte load) per lane and chunk; the dot product masks bit s of every
//    byte in place (DotBits32) and adds 2 * sum - rowsum at the end;
//  * up to 16 tokens: the streaming skinny MFMA kernel of gemm.hip in its
//    1-bit mode (each bit expanded to the byte 2 bit = t + 1 by one shift and
//    one mask per 4 weights, so its epilogue is the 2-bit one);
//  * otherwise: mfma1_kernel, the same MFMA with K walked in segments of 1024
//    whose activations are staged into LDS (double buffered, direct-to-LDS
//    loads) while the previous segment is computed; batches above 64 tokens
//    run as slices of 64.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

struct Gemv1Args {
  const int8_t* xq;
  const float* x_scale;
  const int32_t* rowsum;
  int64_t Kp, Kb;  // padded K of the codes (64) and of the weight rows (128)
  const uint32_t* W;
  const float* w_scale;
  int64_t N;
  float* Y;
  int32_t* acc_out;
};

// LDS byte offset of 16-byte piece p of the activation codes: piece j of the
// 128-byte chunk c = p / 8 sits in slot j ^ (c % 8), so the eight lanes of a
// ds_read_b128 phase (consecutive chunks, same piece) hit eight different
// 16-byte bank groups.
__device__ __forceinline__ int xslot1(int p) {
  const int c = p >> 3;
  return 16 * (8 * c + ((p & 7) ^ (c & 7)));
}

// KC: 128-weight chunks per lane (Kb <= 8192 KC).  R: weight rows per wave.
template <int KC, int R>
__global__ __launch_bounds__(256) void gemv1_kernel(const Gemv1Args a) {
  __shared__ __attribute__((aligned(16))) int8_t xq_lds[8192 * KC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = (int)(a.Kb >> 7);   // 128-weight chunks per row
  const int wpr = (int)(a.Kb >> 5);  // words per row
  const int np = (int)(a.Kp >> 4);   // 16-byte pieces of codes
  const int64_t rb = (int64_t)blockIdx.x * 4 + wave;

  // activation codes before the weights (vmcnt counts in order)
  int4 xi[2 * KC];
  const int4* xg = reinterpret_cast<const int4*>(a.xq);
#pragma unroll
  for (int j = 0; j < 2 * KC; ++j) {
    const int p = tid + 256 * j;
    xi[j] = p < np ? xg[p] : make_int4(0, 0, 0, 0);
  }
  uint4 w[R][KC];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t n = rb * R + r;
    n = n < a.N ? n : a.N - 1;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      int c = lane + 64 * i;
      c = c < C ? c : C - 1;
      w[r][i] = load_stream_u4(reinterpret_cast<const uint4*>(a.W + n * wpr) + c);
    }
  }
  const float sw = a.w_scale[0];
  const float gx = a.x_scale[0];
  const int rsum = a.rowsum[0];
#pragma unroll
  for (int j = 0; j < 2 * KC; ++j) {
    const int p = tid + 256 * j;
    if (p < 8 * C) *reinterpret_cast<int4*>(xq_lds + xslot1(p)) = xi[j];
  }
  __syncthreads();

  int part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) part[r] = 0;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int c = lane + 64 * i;
    if (c < C) {
      int4 x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = *reinterpret_cast<const int4*>(xq_lds + xslot1(8 * c + q));
#pragma unroll
      for (int r = 0; r < R; ++r) {
        DotBits32 d;
        d.add(w[r][i].x, x[0], x[1]);
        d.add(w[r][i].y, x[2], x[3]);
        d.add(w[r][i].z, x[4], x[5]);
        d.add(w[r][i].w, x[6], x[7]);
        part[r] += d.total();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (rb * R >= a.N) return;
  const int sum = wave_transpose_reduce<R>(part);  // sum of q over the +1 weights
  const int row = gemv_row<R>(lane);
  const int64_t n = rb * R + row;
  if (lane < R && n < a.N) {
    const int acc = 2 * sum - rsum;
    a.Y[n] = dequant(acc, __fmul_rn(sw, gx));
    if (a.acc_out) a.acc_out[n] = acc;
  }
}

constexpr int kB1Lpr = 8;                    // lanes per weight row per load (8 x 16 B)
constexpr int kB1Seg = kB1Lpr * 128;         // weights per row per step and K segment
constexpr int kB1Bp = kB1Seg / 8 + 16;       // staged bytes per weight row (+ pad)
constexpr int kB1Pitch = kB1Seg + 16;        // staged activation row (+16 B spreads banks)
constexpr int kB1Wpb = 4;                    // waves (16-row weight tiles) per block

__host__ __device__ constexpr int64_t b1_xbuf_bytes(int tms) {
  return staged_rows_bytes(16 * tms, kB1Pitch);
}
__host__ __device__ constexpr int64_t b1_lds_bytes(int tms) {
  return 2 * b1_xbuf_bytes(tms) + (int64_t)kB1Wpb * 16 * kB1Bp;
}

// Up to 16 TMS tokens (M <= 16 TMS).  Wave w of block b owns weight rows
// 64 b + 16 w .. +15; lane (g, li) of k-step s feeds weights
// 256 blk + 64 g + 16 s .. +15 of row li and the same activation bytes of
// token row 16 tm + li.
template <int TMS>
__global__ __launch_bounds__(64 * kB1Wpb) void mfma1_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int M, int64_t Kp, int64_t Kb,
    const uint32_t* __restrict__ W, const float* __restrict__ w_scale, int64_t N,
    float* __restrict__ Y, int32_t* __restrict__ acc_out) {
  constexpr int RPI = 64 / kB1Lpr;  // rows per load instruction
  constexpr int NI = 16 / RPI;      // load instructions per step
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, li = lane & 15;
  int8_t* xbuf0 = lds;
  int8_t* xbuf1 = lds + b1_xbuf_bytes(TMS);
  int8_t* lds_w = lds + 2 * b1_xbuf_bytes(TMS) + wave * 16 * kB1Bp;
  TokenOperands<TMS> tok;  // the epilogue's scales and row sums, the oldest loads
  tok.load(x_scale, rowsum, M, 0);
  const float sw = w_scale[0];
  const int64_t wpr = Kb / 32;
  const int C = (int)(Kb / 128);  // 16-byte pieces per weight row
  const int nseg = (int)((Kb + kB1Seg - 1) / kB1Seg);
  const int64_t nbase = (int64_t)blockIdx.x * (16 * kB1Wpb) + 16 * wave;
  const int lr = lane / kB1Lpr, lc = lane % kB1Lpr;

  uint4 st[NI];
  auto load_step = [&](int seg) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int64_t n = nbase + RPI * i + lr;
      n = n < N ? n : N - 1;
      const int c = seg * kB1Lpr + lc;
      st[i] = c < C ? load_stream_u4(reinterpret_cast<const uint4*>(W + n * wpr) + c)
                    : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stage_x = [&](int seg) {
    const int64_t k0 = (int64_t)seg * kB1Seg;
    const int64_t rest = Kp - k0;  // codes past Kp read as zero
    const int klen = rest < kB1Seg ? (int)rest : kB1Seg;
    stage_rows_lds<64 * kB1Wpb>(Xq, Kp, M, k0, klen, kB1Pitch, (seg & 1) ? xbuf1 : xbuf0);
  };
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  v4i acc[TMS][2];
#pragma unroll
  for (int tm = 0; tm < TMS; ++tm) acc[tm][0] = acc[tm][1] = v4i{0, 0, 0, 0};

  stage_x(0);
  load_step(0);
  for (int seg = 0; seg < nseg; ++seg) {
    // segment seg's codes and weights have landed; every wave is done with
    // the buffer the next segment overwrites
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (seg + 1 < nseg) stage_x(seg + 1);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      *reinterpret_cast<uint4*>(lds_w + (RPI * i + lr) * kB1Bp + 16 * lc) = st[i];
    wave_sync();
    if (seg + 1 < nseg) load_step(seg + 1);
    const int8_t* xb = (seg & 1) ? xbuf1 : xbuf0;
    const int64_t k0 = (int64_t)seg * kB1Seg;
#pragma unroll
    for (int blk = 0; blk < kB1Seg / 256; ++blk) {
      if (k0 + 256 * blk < Kb) {
        const uint2 bw = *reinterpret_cast<const uint2*>(lds_w + li * kB1Bp + 32 * blk + 8 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const uint32_t wd = s < 2 ? bw.x : bw.y;
          const v4i bv = (s & 1) ? bits_operand<1>(wd) : bits_operand<0>(wd);
#pragma unroll
          for (int tm = 0; tm < TMS; ++tm) {
            const int row = 16 * tm + li;
            const v4i av = row < M ? *reinterpret_cast<const v4i*>(xb + row * kB1Pitch + 256 * blk +
                                                                   64 * g + 16 * s)
                                   : v4i{0, 0, 0, 0};
            acc[tm][s & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc[tm][s & 1], 0, 0, 0);
          }
        }
      }
    }
    wave_sync();
  }

  // result lane l, register r of token tile tm: token 16 tm + 4 g + r, weight row nbase + li
  const int64_t n = nbase + li;
#pragma unroll
  for (int tm = 0; tm < TMS; ++tm)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * tm + 4 * g + r;
      if (m < M && n < N) {
        const int a = acc[tm][0][r] + acc[tm][1][r] - tok.rs[tm][r];
        Y[(int64_t)m * N + n] = dequant_fast(a, __fmul_rn(sw, tok.xs[tm][r]));
        if (acc_out) acc_out[(int64_t)m * N + n] = a;
      }
    }
}

// ---------------------------------------------------------------------------
// Host side.

template <int KC, int R>
static hipError_t gemv1_go(const Gemv1Args& a, hipStream_t s) {
  const int64_t nrb = (a.N + R - 1) / R;
  hipLaunchKernelGGL((gemv1_kernel<KC, R>), dim3((unsigned)((nrb + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int TMS>
static hipError_t mfma1_go(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                           int64_t Kp, int64_t Kb, const uint32_t* Wb, const float* ws, int64_t N,
                           float* Y, int32_t* acc_out, hipStream_t s) {
  static bool once = ((void)hipFuncSetAttribute(reinterpret_cast<const void*>(mfma1_kernel<TMS>),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                (int)b1_lds_bytes(TMS)),
                      true);
  (void)once;
  const unsigned blocks = (unsigned)((N + 16 * kB1Wpb - 1) / (16 * kB1Wpb));
  hipLaunchKernelGGL(mfma1_kernel<TMS>, dim3(blocks), dim3(64 * kB1Wpb), (size_t)b1_lds_bytes(TMS),
                     s, Xq, xs, rs, (int)M, Kp, Kb, Wb, ws, N, Y, acc_out);
  return hipGetLastError();
}

hipError_t launch_forward_1bit(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                               int64_t K, const uint32_t* Wb, const float* ws, int64_t N, float* Y,
                               int32_t* acc_out, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64, Kb = (K + 127) / 128 * 128;
  if (M == 1 && Kb <= 4 * 8192) {
    const Gemv1Args a{Xq, xs, rs, Kp, Kb, Wb, ws, N, Y, acc_out};
    const int64_t C = Kb / 128;
    if (C <= 64) return gemv1_go<1, 4>(a, s);
    if (C <= 128) return gemv1_go<2, 4>(a, s);
    if (C <= 192) return gemv1_go<3, 2>(a, s);
    return gemv1_go<4, 2>(a, s);
  }
  if (stream_1bit_ok(M, K, N)) return launch_stream_1bit(Xq, xs, rs, M, K, Wb, ws, N, Y, acc_out, s);
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int64_t ms = M - m0 < 64 ? M - m0 : 64;
    const int8_t* x = Xq + m0 * Kp;
    float* y = Y + m0 * N;
    int32_t* ao = acc_out ? acc_out + m0 * N : nullptr;
    hipError_t e;
    if (ms <= 16) e = mfma1_go<1>(x, xs + m0, rs + m0, ms, Kp, Kb, Wb, ws, N, y, ao, s);
    else if (ms <= 32) e = mfma1_go<2>(x, xs + m0, rs + m0, ms, Kp, Kb, Wb, ws, N, y, ao, s);
    else if (ms <= 48) e = mfma1_go<3>(x, xs + m0, rs + m0, ms, Kp, Kb, Wb, ws, N, y, ao, s);
    else e = mfma1_go<4>(x, xs + m0, rs + m0, ms, Kp, Kb, Wb, ws, N, y, ao, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace bl

// Decode GEMV (one token) on gfx950: y[n] = dequant(sum_k q[k] * t[n][k]).
//
// dashen-tech "BitNet.cpp 深度解析" §3.1: with ternary weights the product is
// the sum of activations under +1 weights minus the sum under -1 weights.
// Here it is taken in the shifted-code form
//   acc = sum_k q[k] * (t + 1) - sum_k q[k],
// so the 2-bit codes (0, 1, 2) feed the 4-wide int8 dot product directly
// after a mask, and the row sum of q (from the quantiser) removes the shift.
//
// Layout of the work: a wave owns R consecutive weight rows; its 64 lanes
// span K, lane l taking the 64-weight chunks l, l+64, ... (16 bytes of 2-bit
// codes, one dwordx4 load per row and chunk), so each row is read as one
// contiguous stream.  The activation chunk of a lane is the same for every
// row and stays in registers.  The R per-lane partial sums are reduced across
// the wave with a transposing butterfly (R rows in log2(64) steps), and the
// epilogue dequantises: y = ((float)acc * (g_w * g_x)) / 127.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

enum { EPI_STORE = 0, EPI_GATEUP = 1 };

// Reduce v[0..R) (per-lane partials of R rows) across the 64 lanes.  On
// return lane l holds the full sum of row (l >> (6 - log2 R)) in v[0].
template <int R>
__device__ __forceinline__ int wave_transpose_reduce(int (&v)[R]) {
  const int lane = threadIdx.x & 63;
  int cnt = R;
  int o = 32;
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    if (cnt > 1) {
      const int half = cnt >> 1;
      const bool hi = (lane & o) != 0;
#pragma unroll
      for (int i = 0; i < R / 2; ++i) {
        if (i < half) {
          const int keep = hi ? v[half + i] : v[i];
          const int send = hi ? v[i] : v[half + i];
          v[i] = keep + __shfl_xor(send, o);
        }
      }
      cnt = half;
    } else {
      v[0] += __shfl_xor(v[0], o);
    }
    o >>= 1;
  }
  return v[0];
}

// KC: 64-weight chunks per lane per K segment (a segment is 4096 * KC
// weights).  R: rows per wave.
// EPI_STORE: rows n0..n0+R-1 of W -> Y.  EPI_GATEUP: rows n0..n0+R/2-1 of
// Wg and of Wu -> h = relu(g)^2 * u, plus the block's max |h| into
// gh_parts[blockIdx.x].
template <int KC, int R, int EPI>
__global__ __launch_bounds__(256) void gemv_kernel(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int64_t Kp, const uint32_t* __restrict__ W0,
    const float* __restrict__ s0, const uint32_t* __restrict__ W1, const float* __restrict__ s1,
    int64_t N, float* __restrict__ Y, int32_t* __restrict__ acc_out,
    float* __restrict__ gh_parts) {
  constexpr int RW = (EPI == EPI_GATEUP) ? R / 2 : R;  // output rows per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = ((int64_t)blockIdx.x * 4 + wave) * RW;
  const int64_t C = Kp / 64;  // chunks per row
  const int64_t wpr = Kp / 16;

  int part[R];
#pragma unroll
  for (int r = 0; r < R; ++r) part[r] = 0;

  // K is walked in segments of 64*KC chunks (one segment when K <= 4096*KC)
  for (int64_t seg = 0; seg < C; seg += 64 * KC) {
    // activation chunks of this lane, natural order: 16 x int32 per chunk
    int x[KC][16];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int64_t c = seg + lane + 64 * i;
      if (c < C) {
        const int4* p = reinterpret_cast<const int4*>(xq + 64 * c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int4 v = p[q];
          x[i][4 * q + 0] = v.x; x[i][4 * q + 1] = v.y; x[i][4 * q + 2] = v.z; x[i][4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q) x[i][q] = 0;
      }
    }

    // weight chunks: row r of this wave, chunk i
    uint4 w[R][KC];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint32_t* base;
      int64_t n;
      if constexpr (EPI == EPI_GATEUP) {
        n = n0 + (r % RW);
        base = (r < RW) ? W0 : W1;
      } else {
        n = n0 + r;
        base = W0;
      }
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const int64_t c = seg + lane + 64 * i;
        if (n < N && c < C)
          w[r][i] = *reinterpret_cast<const uint4*>(base + n * wpr + 4 * c);
        else
          w[r][i] = make_uint4(0u, 0u, 0u, 0u);
      }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      Dot16 d;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        d.add(w[r][i].x, x[i][0], x[i][1], x[i][2], x[i][3]);
        d.add(w[r][i].y, x[i][4], x[i][5], x[i][6], x[i][7]);
        d.add(w[r][i].z, x[i][8], x[i][9], x[i][10], x[i][11]);
        d.add(w[r][i].w, x[i][12], x[i][13], x[i][14], x[i][15]);
      }
      part[r] += d.total();
    }
  }

  const int sum = wave_transpose_reduce<R>(part);
  constexpr int LOGR = (R == 1) ? 0 : (R == 2) ? 1 : (R == 4) ? 2 : 3;
  const int row = lane >> (6 - LOGR);
  const bool leader = (lane & ((64 >> LOGR) - 1)) == 0;
  const int acc = sum - rowsum[0];

  if constexpr (EPI == EPI_STORE) {
    const int64_t n = n0 + row;
    if (leader && n < N) {
      const float sc = __fmul_rn(s0[0], x_scale[0]);
      Y[n] = dequant(acc, sc);
      if (acc_out) acc_out[n] = acc;
    }
  } else {
    // rows [0, RW) are gate, [RW, R) are up; bring up's sum next to gate's
    constexpr int SPAN = 64 >> LOGR;  // lanes per row
    const int acc_up = __shfl(acc, (lane + RW * SPAN) & 63);
    float hmax = 0.0f;
    const int64_t n = n0 + row;
    if (leader && row < RW && n < N) {
      const float g = dequant(acc, __fmul_rn(s0[0], x_scale[0]));
      const float u = dequant(acc_up, __fmul_rn(s1[0], x_scale[0]));
      const float a = g > 0.0f ? g : 0.0f;
      const float h = __fmul_rn(__fmul_rn(a, a), u);
      Y[n] = h;
      hmax = fabsf(h);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, o));
    __shared__ float red[4];
    if (lane == 0) red[wave] = hmax;
    __syncthreads();
    if (threadIdx.x == 0)
      gh_parts[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
}

template <int R, int EPI>
static hipError_t gemv_dispatch(const int8_t* xq, const float* xs, const int32_t* rs, int64_t Kp,
                                const uint32_t* W0, const float* s0, const uint32_t* W1,
                                const float* s1, int64_t N, float* Y, int32_t* acc_out,
                                float* gh_parts, hipStream_t s) {
  constexpr int RW = (EPI == EPI_GATEUP) ? R / 2 : R;
  const int64_t C = Kp / 64;
  const unsigned blocks = (unsigned)((N + 4 * RW - 1) / (4 * RW));
#define BL_GEMV_CASE(KCV)                                                                     \
  hipLaunchKernelGGL((gemv_kernel<KCV, R, EPI>), dim3(blocks), dim3(256), 0, s, xq, xs, rs, Kp, \
                     W0, s0, W1, s1, N, Y, acc_out, gh_parts)
  if (C <= 64) BL_GEMV_CASE(1);
  else if (C <= 128) BL_GEMV_CASE(2);
  else if (C <= 192) BL_GEMV_CASE(3);
  else BL_GEMV_CASE(4);
#undef BL_GEMV_CASE
  return hipGetLastError();
}

hipError_t launch_gemv(const int8_t* xq, const float* xs, const int32_t* rs, int64_t K,
                       const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                       int32_t* acc_out, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  return gemv_dispatch<4, EPI_STORE>(xq, xs, rs, Kp, Wp, ws, nullptr, nullptr, N, Y, acc_out,
                                     nullptr, s);
}

int64_t gemv_gateup_parts(int64_t N) { return (N + 7) / 8; }

hipError_t launch_gemv_gateup(const int8_t* xq, const float* xs, const int32_t* rs, int64_t K,
                              const uint32_t* Wg, const float* sg, const uint32_t* Wu,
                              const float* su, int64_t N, float* H, float* gh_parts,
                              int* nparts, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  *nparts = (int)gemv_gateup_parts(N);
  return gemv_dispatch<4, EPI_GATEUP>(xq, xs, rs, Kp, Wg, sg, Wu, su, N, H, nullptr, gh_parts, s);
}

}  // namespace bl

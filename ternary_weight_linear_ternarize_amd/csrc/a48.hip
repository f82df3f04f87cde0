// BitNet a4.8 activations (youngju.dev "BitNet論文分析", section "BitNet
// a4.8"): the top fraction of each token's activations is split off and kept
// in 8 bits, the rest is quantised to 4 bits.
//
// Reading taken here: per token row the n_out entries of largest |x|
// (ties to the lower index) are the outliers, quantised like the int8
// activation quantiser (Q = 127) with their own scale g8 = max |x| over them;
// every other entry is quantised with Q = 7 (symmetric 4-bit range) and
// g4 = max |x| over the rest.  Both code vectors are stored as int8 rows of
// Kp bytes, each zero where the other holds the entry, so the product is two
// ternary x int8 products,
//   y = (acc4 * (g_w g4)) / 7 + (acc8 * (g_w g8)) / 127.
//
//  * a48_quant_kernel: one block per row; the n_out-th largest |x| is found by
//    an MSB-first radix select on the bits of |x| (digits of 12, 12 and 7
//    bits, LDS histograms), ties at the threshold are taken in index order
//    through a block prefix count;
//  * gemv_a48_kernel (one token): the GEMV of gemv.hip with both code
//    vectors in LDS and the masked weight fields shared by the two dot
//    products (Dot16x2);
//  * more tokens: the product kernels run with their int32 accumulators kept
//    (once over both code matrices when they are stacked and 2M <= 16, else
//    once per code matrix), then a48_combine_kernel forms y; where the
//    stacked product runs on the streaming kernel, its epilogue forms y and
//    there is no combine launch.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

// Exclusive prefix sum of one int per thread in thread order (NT threads);
// *total receives the block sum.  sh holds NT / 64 ints.
template <int NT>
__device__ int block_excl_scan(int v, int* sh, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(inc, o);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int s = sh[w];
    if (w < wave) base += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Inclusive prefix sum over the 64 lanes of a wave (row shifts within rows
// of 16 lanes, then the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp::mov<0x111>(0, x);
  x += dpp::mov<0x112>(0, x);
  x += dpp::mov<0x114>(0, x);
  x += dpp::mov<0x118>(0, x);
  x += dpp::mov<dpp::kBcast15, 0xA>(0, x);
  x += dpp::mov<dpp::kBcast31, 0xC>(0, x);
  return x;
}

__device__ __forceinline__ int a48_code(float x, float q, float d) {
  float r = __builtin_rintf(__fdiv_rn(__fmul_rn(x, q), d));
  r = fminf(fmaxf(r, -q), q);
  return (int)r;
}

// The same code with the division by d done by Markstein's correction from
// y = RN(1/d) (as quant_code_fast): RN(q0 + r y) with q0 = RN(a y) and the
// exact residual r = a - q0 d is the correctly rounded a / d while d and 1/d
// are normal (fast rows: 1e-5 <= d < 2^100); a / d only matters near k + 1/2,
// where a is normal.
__device__ __forceinline__ int a48_code_fast(float x, float q, float d, float y) {
  const float a = __fmul_rn(x, q);
  const float q0 = __fmul_rn(a, y);
  const float r = __builtin_fmaf(-q0, d, a);
  float v = __builtin_rintf(__builtin_fmaf(r, y, q0));
  v = fminf(fmaxf(v, -q), q);
  return (int)v;
}

// Thread t owns indices t E .. t E + E - 1 (index order = thread order).
//
// The n_out-th largest key T (key = the bits of |x|, bit 31 clear) is found
// digit by digit, bits 30..19, 18..7 and 6..0: every thread adds its
// keys that match the digits found so far to an LDS histogram of the next
// digit; wave 0 then scans that histogram from the top (each lane sums a run
// of bins, a wave prefix sum picks the run, its lane walks it) while the
// other waves clear the histogram the next digit uses.  Two barriers per
// digit.  Keys equal to T are outliers in index order up to the number still
// needed; the block prefix count that ranks them runs only when the keys
// equal to T are more than that.
template <bool BF16, int E>
__global__ __launch_bounds__(1024) void a48_quant_kernel(const void* __restrict__ X, int64_t K,
                                                         int64_t Kp, int n_out,
                                                         int8_t* __restrict__ Xq4,
                                                         float* __restrict__ g4o,
                                                         int32_t* __restrict__ rs4o,
                                                         int8_t* __restrict__ Xq8,
                                                         float* __restrict__ g8o,
                                                         int32_t* __restrict__ rs8o) {
  constexpr int NT = 1024, NW = NT / 64, HB = 4096;
  __shared__ __attribute__((aligned(16))) int hist[2][HB];
  __shared__ int shi[2][NW];
  __shared__ float shf[2][NW];
  __shared__ int sel[3];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t m = blockIdx.x;
  const int64_t k0 = (int64_t)tid * E;
  const char* row = reinterpret_cast<const char*>(X) + m * K * (BF16 ? 2 : 4);

  float v[E];
  const bool vec = k0 + E <= K && (reinterpret_cast<uintptr_t>(row) & (BF16 ? 7 : 15)) == 0;
  if (vec) {
    // E / 4 loads of 4 consecutive values (the row start is aligned)
#pragma unroll
    for (int j = 0; j < E / 4; ++j) {
      if constexpr (BF16) {
        const uint2 u = reinterpret_cast<const uint2*>(row)[k0 / 4 + j];
        v[4 * j + 0] = __uint_as_float(u.x << 16);
        v[4 * j + 1] = __uint_as_float(u.x & 0xffff0000u);
        v[4 * j + 2] = __uint_as_float(u.y << 16);
        v[4 * j + 3] = __uint_as_float(u.y & 0xffff0000u);
      } else {
        const float4 f = reinterpret_cast<const float4*>(row)[k0 / 4 + j];
        v[4 * j + 0] = f.x;
        v[4 * j + 1] = f.y;
        v[4 * j + 2] = f.z;
        v[4 * j + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = (k0 + e < K) ? load_act<BF16>(row, k0 + e) : 0.0f;
  }
  auto key = [&](int e) { return __float_as_uint(v[e]) & 0x7fffffffu; };

  const int nsel = n_out < K ? n_out : (int)K;
  uint32_t T = 0u, pmask = 0u;
  int need = nsel, nties = 0;
  if (nsel > 0 && nsel < K) {
    for (int i = tid; i < 2 * HB; i += NT) (&hist[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int shift = p == 0 ? 19 : p == 1 ? 7 : 0;
      const int nb = p == 2 ? 128 : 4096;
      int* h = hist[p & 1];
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (k0 + e < K && (key(e) & pmask) == T)
          atomicAdd(&h[(key(e) >> shift) & (uint32_t)(nb - 1)], 1);
      __syncthreads();
      if (wave == 0) {
        // lane l sums bins nb-1-l*per down to nb-(l+1)*per; a wave prefix sum
        // picks the lane whose run holds the need-th key from the top, then
        // that run is spread over the lanes (one bin each) and scanned again
        const int per = nb / 64;
        const int lo = nb - (lane + 1) * per;
        int run = 0;
        if (per >= 4) {
          const int4* hp = reinterpret_cast<const int4*>(h + lo);
          for (int j = 0; j < per / 4; ++j) {
            const int4 q = hp[j];
            run += q.x + q.y + q.z + q.w;
          }
        } else {
          for (int j = 0; j < per; ++j) run += h[lo + j];
        }
        const int inc = wave_incl_scan(run);
        const uint64_t hit = __ballot(inc - run < need && need <= inc);
        const int L = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
        const int base = __builtin_amdgcn_readlane(inc - run, L);
        const int top = nb - 1 - L * per;
        const int c = lane < per ? h[top - lane] : 0;
        const int inc2 = wave_incl_scan(c) + base;
        const uint64_t hit2 = __ballot(inc2 - c < need && need <= inc2);
        const int J = __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit2));
        if (lane == J) {
          sel[0] = top - J;
          sel[1] = inc2 - c;
          sel[2] = c;
        }
      } else if (p == 1) {
        // the last digit counts into hist[0] again
        for (int i = tid - 64; i < HB; i += NT - 64) hist[0][i] = 0;
      }
      __syncthreads();
      T |= (uint32_t)sel[0] << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      need -= sel[1];
      nties = sel[2];
    }
  }

  bool out[E];
  if (nsel >= K) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = k0 + e < K;
  } else if (nsel == 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = false;
  } else if (nties == need) {
    // every key equal to T is an outlier
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = k0 + e < K && key(e) >= T;
  } else {
    int eq = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) eq += (k0 + e < K && key(e) == T) ? 1 : 0;
    int tot;
    int r = block_excl_scan<NT>(eq, &shi[0][0], &tot);  // rank of this thread's first tie
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool real = k0 + e < K;
      const bool tie = real && key(e) == T;
      out[e] = real && (key(e) > T || (tie && r < need));
      r += tie ? 1 : 0;
    }
  }

  // both scales in one block reduction
  float a8 = 0.0f, a4 = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const float a = fabsf(v[e]);
    if (out[e]) a8 = fmaxf(a8, a);
    else a4 = fmaxf(a4, a);
  }
  a8 = dpp::max_nonneg_f32(a8);
  a4 = dpp::max_nonneg_f32(a4);
  if (lane == 0) {
    shf[0][wave] = a8;
    shf[1][wave] = a4;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    a8 = fmaxf(a8, shf[0][w]);
    a4 = fmaxf(a4, shf[1][w]);
  }
  const float d8 = __fadd_rn(a8, kEps), d4 = __fadd_rn(a4, kEps);
  const float y8 = __fdiv_rn(1.0f, d8), y4 = __fdiv_rn(1.0f, d4);
  const bool fast = d8 < 0x1p100f && d4 < 0x1p100f;

  int s4 = 0, s8 = 0;
  uint32_t w4[E / 4], w8[E / 4];
#pragma unroll
  for (int j = 0; j < E / 4; ++j) w4[j] = w8[j] = 0u;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int c4 = 0, c8 = 0;
    if (k0 + e < K) {
      if (fast) {
        if (out[e]) c8 = a48_code_fast(v[e], kQ, d8, y8);
        else c4 = a48_code_fast(v[e], 7.0f, d4, y4);
      } else {
        if (out[e]) c8 = a48_code(v[e], kQ, d8);
        else c4 = a48_code(v[e], 7.0f, d4);
      }
    }
    s4 += c4;
    s8 += c8;
    w4[e / 4] |= (uint32_t)(c4 & 0xff) << (8 * (e % 4));
    w8[e / 4] |= (uint32_t)(c8 & 0xff) << (8 * (e % 4));
  }
#pragma unroll
  for (int j = 0; j < E / 4; ++j) {
    const int64_t k = k0 + 4 * j;
    if (k < Kp) {
      *reinterpret_cast<uint32_t*>(Xq4 + m * Kp + k) = w4[j];
      *reinterpret_cast<uint32_t*>(Xq8 + m * Kp + k) = w8[j];
    }
  }
  // both row sums in one block reduction (shi[1] is not in use by the tie scan)
  s4 = dpp::sum_i32(s4);
  s8 = dpp::sum_i32(s8);
  if (lane == 0) {
    shi[0][wave] = s4;
    shi[1][wave] = s8;
  }
  __syncthreads();
  if (tid == 0) {
    int t4 = 0, t8 = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      t4 += shi[0][w];
      t8 += shi[1][w];
    }
    g4o[m] = a4;
    g8o[m] = a8;
    rs4o[m] = t4;
    rs8o[m] = t8;
  }
}

struct A48Args {
  const int8_t* x4;
  const int8_t* x8;
  const float* g4;
  const float* g8;
  const int32_t* rs4;
  const int32_t* rs8;
  int64_t Kp;
  const uint32_t* W;
  const float* w_scale;
  int64_t N;
  float* Y;
  int32_t* acc;  // optional: acc4 [N] then acc8 [N]
};

// KC: 64-weight chunks per lane (Kp <= 4096 KC).  R: weight rows per wave.
template <int KC, int R>
__global__ __launch_bounds__(256) void gemv_a48_kernel(const A48Args a) {
  __shared__ __attribute__((aligned(16))) int8_t q4_lds[4096 * KC];
  __shared__ __attribute__((aligned(16))) int8_t q8_lds[4096 * KC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = (int)(a.Kp >> 6);
  const int wpr = (int)(a.Kp >> 4);
  const int64_t rb = (int64_t)blockIdx.x * 4 + wave;

  int4 x4[KC], x8[KC];
  const int4* g4p = reinterpret_cast<const int4*>(a.x4);
  const int4* g8p = reinterpret_cast<const int4*>(a.x8);
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int p = tid + 256 * j;
    x4[j] = p < 4 * C ? g4p[p] : make_int4(0, 0, 0, 0);
    x8[j] = p < 4 * C ? g8p[p] : make_int4(0, 0, 0, 0);
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
  const float s4 = __fmul_rn(sw, a.g4[0]), s8 = __fmul_rn(sw, a.g8[0]);
  const int r4 = a.rs4[0], r8 = a.rs8[0];
#pragma unroll
  for (int j = 0; j < KC; ++j) {
    const int p = tid + 256 * j;
    if (p < 4 * C) {
      *reinterpret_cast<int4*>(q4_lds + xslot(p)) = x4[j];
      *reinterpret_cast<int4*>(q8_lds + xslot(p)) = x8[j];
    }
  }
  __syncthreads();

  int p4[R], p8[R];
#pragma unroll
  for (int r = 0; r < R; ++r) p4[r] = p8[r] = 0;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int c = lane + 64 * i;
    if (c < C) {
      int4 u[4], z[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u[q] = *reinterpret_cast<const int4*>(q4_lds + xslot(4 * c + q));
        z[q] = *reinterpret_cast<const int4*>(q8_lds + xslot(4 * c + q));
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        Dot16x2 d;
        d.add(w[r][i].x, u[0], z[0]);
        d.add(w[r][i].y, u[1], z[1]);
        d.add(w[r][i].z, u[2], z[2]);
        d.add(w[r][i].w, u[3], z[3]);
        p4[r] += d.x.total();
        p8[r] += d.z.total();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (rb * R >= a.N) return;
  const int t4 = wave_transpose_reduce<R>(p4);
  const int t8 = wave_transpose_reduce<R>(p8);
  const int row = gemv_row<R>(lane);
  const int64_t n = rb * R + row;
  if (lane < R && n < a.N) {
    const int acc4 = t4 - r4, acc8 = t8 - r8;
    a.Y[n] = a48_dequant(acc4, s4, acc8, s8);
    if (a.acc) {
      a.acc[n] = acc4;
      a.acc[a.N + n] = acc8;
    }
  }
}

__global__ __launch_bounds__(256) void a48_combine_kernel(const int32_t* __restrict__ acc,
                                                          const float* __restrict__ g4,
                                                          const float* __restrict__ g8,
                                                          const float* __restrict__ w_scale,
                                                          int64_t M, int64_t N,
                                                          float* __restrict__ Y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * N) return;
  const int64_t m = i / N;
  const float sw = w_scale[0];
  Y[i] = a48_dequant(acc[i], __fmul_rn(sw, g4[m]), acc[M * N + i], __fmul_rn(sw, g8[m]));
}

// ---------------------------------------------------------------------------
// Host side.

template <bool BF16>
static hipError_t a48_quant_go(const void* X, int64_t M, int64_t K, int64_t Kp, int n_out,
                               int8_t* q4, float* g4, int32_t* rs4, int8_t* q8, float* g8,
                               int32_t* rs8, hipStream_t s) {
#define BL_A48Q(E)                                                                               \
  hipLaunchKernelGGL((a48_quant_kernel<BF16, E>), dim3((unsigned)M), dim3(1024), 0, s, X, K, Kp, \
                     n_out, q4, g4, rs4, q8, g8, rs8)
  if (Kp <= 4096) BL_A48Q(4);
  else if (Kp <= 8192) BL_A48Q(8);
  else if (Kp <= 16384) BL_A48Q(16);
  else if (Kp <= 32768) BL_A48Q(32);
  else BL_A48Q(64);
#undef BL_A48Q
  return hipGetLastError();
}

hipError_t launch_act_quant_a48(const void* X, bool bf16, int64_t M, int64_t K, int64_t n_out,
                                int8_t* q4, float* g4, int32_t* rs4, int8_t* q8, float* g8,
                                int32_t* rs8, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  const int no = (int)(n_out < K ? n_out : K);
  return bf16 ? a48_quant_go<true>(X, M, K, Kp, no, q4, g4, rs4, q8, g8, rs8, s)
              : a48_quant_go<false>(X, M, K, Kp, no, q4, g4, rs4, q8, g8, rs8, s);
}

template <int KC, int R>
static hipError_t gemv_a48_go(const A48Args& a, hipStream_t s) {
  const int64_t nrb = (a.N + R - 1) / R;
  hipLaunchKernelGGL((gemv_a48_kernel<KC, R>), dim3((unsigned)((nrb + 3) / 4)), dim3(256), 0, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_forward_a48(const int8_t* x4, const float* g4, const int32_t* rs4,
                              const int8_t* x8, const float* g8, const int32_t* rs8, int64_t M,
                              int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                              int32_t* acc, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  const int64_t C = Kp / 64;
  if (M == 1 && C <= 256) {
    const A48Args a{x4, x8, g4, g8, rs4, rs8, Kp, Wp, ws, N, Y, acc};
    if (C <= 64) return gemv_a48_go<1, 4>(a, s);
    if (C <= 128) return gemv_a48_go<2, 4>(a, s);
    return gemv_a48_go<4, 2>(a, s);
  }
  hipError_t e;
  const bool stacked = x8 == x4 + M * Kp && g8 == g4 + M && rs8 == rs4 + M;
  if (stacked && stream_a48_ok(2 * M, K, N))
    return launch_stream_a48(x4, g4, rs4, 2 * M, K, Wp, ws, N, Y, acc, s);
  if (2 * M <= 16 && stacked) {
    // codes, scales and row sums stacked (the int8 rows right after the int4
    // rows): one product over 2M rows streams the weights once, and its
    // accumulators land as acc4 then acc8
    e = launch_mfma(x4, g4, rs4, 2 * M, K, Wp, ws, N, nullptr, acc, false, s);
  } else {
    // two products with their accumulators kept
    e = launch_mfma(x4, g4, rs4, M, K, Wp, ws, N, Y, acc, false, s);
    if (e == hipSuccess) e = launch_mfma(x8, g8, rs8, M, K, Wp, ws, N, Y, acc + M * N, false, s);
  }
  if (e != hipSuccess) return e;
  const int64_t total = M * N;
  hipLaunchKernelGGL(a48_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                     acc, g4, g8, ws, M, N, Y);
  return hipGetLastError();
}

}  // namespace bl

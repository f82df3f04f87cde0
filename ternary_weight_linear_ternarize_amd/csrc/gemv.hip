// Decode GEMV (one token) on gfx950: y[n] = dequant(sum_k q[k] * t[n][k]).
//
// dashen-tech "BitNet.cpp 深度解析" §3.1: with ternary weights the product is
// the sum of activations under +1 weights minus the sum under -1 weights.
// Here it is taken in the shifted-code form
//   acc = sum_k q[k] * (t + 1) - sum_k q[k],
// so the 2-bit codes (0, 1, 2) feed the 4-wide int8 dot product directly
// after a mask, and the row sum of q removes the shift.
//
// Work layout: a wave owns R consecutive weight rows; its 64 lanes span K,
// lane l taking the 64-weight chunks l, l+64, ... (16 bytes of 2-bit codes:
// one dwordx4 load per row and chunk), so each row is one contiguous stream
// and a wave-wide load covers up to 1 KiB.  All weight loads of a wave are
// issued before anything waits on them.  The activation codes are staged
// once per block in LDS and read chunk by chunk (64 bytes per lane, the same
// for every row), which keeps the register count low enough for every wave of
// a large layer to be resident at once.  The R per-lane partial sums
// are reduced across the wave with a transposing butterfly, and the epilogue
// dequantises: y = ((float)acc * (g_w * g_x)) / 127.
//
// Activation sources (XSRC):
//   XS_INT8  int8 codes, scale and row sum from bitlinear_quant_act;
//   XS_F32 / XS_BF16  float activations quantised inside the kernel (youngju.dev
//            "BitNet b1.58" activation_quant: scale = max |x|, codes
//            rne(x * 127 / (scale + 1e-5))), every block redoing the row
//            (identical bits) into LDS -- one launch per layer;
//   XS_PARTS float activations whose scale is the maximum of per-block partial
//            maxima written by the previous kernel (the FFN's h);
//   XS_NF32 / XS_NBF16  float activations RMS-normalised, then quantised, in
//            every block (the FFN's input: youngju.dev "BitNet b1.58" normalises
//            before activation_quant) -- the norm, the quantiser and the
//            gate/up product in one launch.
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

enum { EPI_STORE = 0, EPI_GATEUP = 1 };
enum { XS_INT8 = 0, XS_F32 = 1, XS_BF16 = 2, XS_PARTS = 3, XS_NF32 = 4, XS_NBF16 = 5 };

constexpr int kFusedMaxKp = 7168;  // largest padded K quantised inside the GEMV
constexpr int kGpPerThread = 2;     // XS_PARTS: partial maxima loaded per thread up front

// Block maximum (non-negative values) / sum over NW waves; red holds NW slots.
template <int NW>
__device__ __forceinline__ float block_maxw(float v, float* red) {
  v = dpp::max_nonneg_f32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = fmaxf(r, red[w]);
  return r;
}

template <int NW>
__device__ __forceinline__ int block_sumw(int v, int* red) {
  v = dpp::sum_i32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r += red[w];
  return r;
}

struct GemvArgs {
  const void* x;            // int8 codes (XS_INT8) or float/bf16 activations
  const float* x_scale;     // XS_INT8: scale g_x
  const int32_t* rowsum;    // XS_INT8: row sum of the codes
  const float* gparts;      // XS_PARTS: partial maxima [nparts]
  int nparts;
  int64_t K, Kp;
  const uint32_t* W0;
  const float* s0;
  const uint32_t* W1;       // EPI_GATEUP: up weights
  const float* s1;
  int64_t N;
  float* Y;
  int32_t* acc_out;         // optional
  float* gh_parts;          // EPI_GATEUP: per-block max |h|
  const float* norm_w;      // XS_NF32/XS_NBF16: RMSNorm weight (NULL: ones)
  float eps;                // XS_NF32/XS_NBF16: RMSNorm epsilon
  float* xn_out;            // XS_NF32/XS_NBF16: optional copy of the normalised row
  int8_t* xq_out;           // fused: optional copy of the codes (block 0)
  float* xs_out;            // fused: optional scale
  int32_t* rs_out;          // fused: optional row sum
};

// Loads the packed chunks of row block rb (clamped into range: straight-line).
template <int KC, int R, int EPI>
__device__ __forceinline__ void gemv_load_w(const GemvArgs& a, int64_t rb, int lane, int C,
                                            int wpr, uint4 (&w)[R][KC]) {
  constexpr int RW = (EPI == EPI_GATEUP) ? R / 2 : R;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t* base = (EPI == EPI_GATEUP && r >= RW) ? a.W1 : a.W0;
    int64_t n = rb * RW + (r % RW);
    n = n < a.N ? n : a.N - 1;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      int c = lane + 64 * i;
      c = c < C ? c : C - 1;
      w[r][i] = load_stream_u4(reinterpret_cast<const uint4*>(base + n * wpr) + c);
    }
  }
}

// Partial dot products of this lane's chunks (lane, lane + 64, ...) with the
// codes in LDS.
template <int KC, int R>
__device__ __forceinline__ void gemv_dots(const uint4 (&w)[R][KC], const int8_t* xq_lds, int lane,
                                          int C, int (&part)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) part[r] = 0;
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    const int c = lane + 64 * i;
    int4 xv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      xv[q] = c < C ? *reinterpret_cast<const int4*>(xq_lds + xslot(4 * c + q))
                    : make_int4(0, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      Dot16 d;
      d.add(w[r][i].x, xv[0].x, xv[0].y, xv[0].z, xv[0].w);
      d.add(w[r][i].y, xv[1].x, xv[1].y, xv[1].z, xv[1].w);
      d.add(w[r][i].z, xv[2].x, xv[2].y, xv[2].z, xv[2].w);
      d.add(w[r][i].w, xv[3].x, xv[3].y, xv[3].z, xv[3].w);
      part[r] += d.total();
    }
    // one chunk of codes live at a time (keeps the register count down)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The same with the codes of this lane's chunks in registers.
template <int KC, int R>
__device__ __forceinline__ void gemv_dots_regs(const uint4 (&w)[R][KC], const int (&x)[KC][16],
                                               int (&part)[R]) {
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
    part[r] = d.total();
  }
}

// Reduce, dequantise and store the rows of row block rb.  Returns this
// lane's max |h| contribution (EPI_GATEUP) or 0.
template <int R, int EPI>
__device__ __forceinline__ float gemv_epilogue(const GemvArgs& a, int64_t rb, int (&part)[R],
                                               int rsum, float gx, float sw0, float sw1) {
  constexpr int RW = (EPI == EPI_GATEUP) ? R / 2 : R;
  const int lane = threadIdx.x & 63;
  const int sum = wave_transpose_reduce<R>(part);
  const int row = gemv_row<R>(lane);
  const bool leader = lane < R;  // one lane per row
  const int acc = sum - rsum;
  const int64_t n = rb * RW + row;
  if constexpr (EPI == EPI_STORE) {
    if (leader && n < a.N) {
      a.Y[n] = dequant(acc, __fmul_rn(sw0, gx));
      if (a.acc_out) a.acc_out[n] = acc;
    }
    return 0.0f;
  } else {
    // rows [0, RW) are gate, [RW, R) are up: up row g + RW sits in the lane
    // next to gate row g (row index g + RW bit-reversed differs in bit 0)
    const int acc_up = dpp::xchg<1>(acc);
    float hm = 0.0f;
    if (leader && row < RW && n < a.N) {
      const float gv = dequant(acc, __fmul_rn(sw0, gx));
      const float uv = dequant(acc_up, __fmul_rn(sw1, gx));
      const float r = gv > 0.0f ? gv : 0.0f;
      const float h = __fmul_rn(__fmul_rn(r, r), uv);
      a.Y[n] = h;
      hm = fabsf(h);
    }
    return hm;
  }
}

// KC: 64-weight chunks per lane (Kp <= 4096 * KC).  R: weight rows per wave
// (one row block per wave: every load of the grid is in flight at once, the
// pattern that measured fastest for both small and large matrices).
template <int KC, int R, int EPI, int XSRC, int NT>
__global__ __launch_bounds__(NT) void gemv_kernel(const GemvArgs a) {
  constexpr int RW = (EPI == EPI_GATEUP) ? R / 2 : R;  // output rows per wave
  constexpr bool FUSED = XSRC != XS_INT8;
  constexpr bool NORM = XSRC == XS_NF32 || XSRC == XS_NBF16;
  constexpr bool BF = XSRC == XS_BF16 || XSRC == XS_NBF16;
  constexpr int NW = NT / 64;  // waves per block
  __shared__ __attribute__((aligned(16))) int8_t xq_lds[4096 * KC];
  __shared__ float redf[NW];
  __shared__ int redi[NW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = (int)(a.Kp >> 6);  // 64-weight chunks per row
  const int wpr = (int)(a.Kp >> 4);
  const int64_t rb = (int64_t)blockIdx.x * NW + wave;  // this wave's row block

  // Activation loads are issued before the weight loads: vmcnt counts in
  // order, so waiting for the activations then leaves the weights in flight
  // and the staging/quantisation below overlaps the weight stream.
  constexpr int NWT = 1024 * KC / NT;  // fused: words per thread (Kp <= 4096 * KC)
  constexpr int NXI = (256 * KC + NT - 1) / NT;  // int8: 16-byte pieces per thread
  int4 xi[NXI];
  float xv[NWT][4];
  float nwv[NORM ? NWT : 1][4];  // NORM: the norm weights of this thread's words
  float g = 0.0f;
  uint32_t gp[kGpPerThread] = {};  // XS_PARTS: partial maxima (float bits)
  if constexpr (!FUSED) {
    const int4* xg = reinterpret_cast<const int4*>(a.x);
#pragma unroll
    for (int j = 0; j < NXI; ++j) {
      const int p = tid + NT * j;
      xi[j] = p < 4 * C ? xg[p] : make_int4(0, 0, 0, 0);
    }
  } else {
    const int K = (int)a.K, nw = (int)(a.Kp >> 2);
    if constexpr (XSRC == XS_PARTS) {
      // the partial maxima: branch-free loads of kGpPerThread per thread
      // (past nparts they read 0), so they are in flight together with the
      // row and the weights instead of ahead of them; any beyond that in a loop
      const buf_rsrc rg = make_buf_rsrc(a.gparts, (uint32_t)(4 * a.nparts));
#pragma unroll
      for (int i = 0; i < kGpPerThread; ++i)
        gp[i] = __builtin_amdgcn_raw_buffer_load_b32(rg, (uint32_t)(4 * (tid + NT * i)), 0, 0);
      for (int p = tid + NT * kGpPerThread; p < a.nparts; p += NT) g = fmaxf(g, a.gparts[p]);
    }
    const bool vec = (reinterpret_cast<uintptr_t>(a.x) & (BF ? 7 : 15)) == 0;
#pragma unroll
    for (int j = 0; j < NWT; ++j) {
      const int wd = tid + NT * j;
      if (vec && 4 * wd + 3 < K) {
        if constexpr (BF) {
          const uint2 u = reinterpret_cast<const uint2*>(a.x)[wd];
          xv[j][0] = __uint_as_float(u.x << 16);
          xv[j][1] = __uint_as_float(u.x & 0xffff0000u);
          xv[j][2] = __uint_as_float(u.y << 16);
          xv[j][3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
          const float4 f = reinterpret_cast<const float4*>(a.x)[wd];
          xv[j][0] = f.x; xv[j][1] = f.y; xv[j][2] = f.z; xv[j][3] = f.w;
        }
      } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int k = 4 * wd + b;
          xv[j][b] = (wd < nw && k < K) ? load_act<BF>(a.x, k) : 0.0f;
        }
      }
    }
    if constexpr (NORM) {
      // the norm weights (if any) ride with the row, as buffer loads that
      // read 0 past K, instead of being fetched after the mean square
      if (a.norm_w) {
        const buf_rsrc rw = make_buf_rsrc(a.norm_w, (uint32_t)(4 * K));
#pragma unroll
        for (int j = 0; j < NWT; ++j)
#pragma unroll
          for (int b = 0; b < 4; ++b)
            nwv[j][b] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rw, (uint32_t)(4 * (4 * (tid + NT * j) + b)), 0, 0));
      }
    }
  }

  uint4 w[R][KC];
  gemv_load_w<KC, R, EPI>(a, rb, lane, C, wpr, w);

  const float sw0 = a.s0[0];
  const float sw1 = (EPI == EPI_GATEUP) ? a.s1[0] : 0.0f;
  float gx = 0.0f;
  int rsum = 0;
  if constexpr (!FUSED) {
    gx = a.x_scale[0];
    rsum = a.rowsum[0];
#pragma unroll
    for (int j = 0; j < NXI; ++j) {
      const int p = tid + NT * j;
      if (p < 4 * C) *reinterpret_cast<int4*>(xq_lds + xslot(p)) = xi[j];
    }
    __syncthreads();
  } else {
    // quantise the whole row into LDS (every block does the same, same bits)
    const int nw = (int)(a.Kp >> 2);
    if constexpr (NORM) {
      // xn = (x * r) * w, r = 1 / sqrt(ms + eps), ms from the exact sum of
      // squares (block_meansq); the padding words stay zero
      __shared__ SumsqScratch sh;
      const int K = (int)a.K;
      const float ms = block_meansq<NWT, NT>(xv, a.K, sh);
      const float r = __fdiv_rn(1.0f, __builtin_sqrtf(__fadd_rn(ms, a.eps)));
#pragma unroll
      for (int j = 0; j < NWT; ++j) {
        const int wd = tid + NT * j;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int k = 4 * wd + b;
          const bool in = wd < nw && k < K;
          float v = __fmul_rn(xv[j][b], r);
          if (a.norm_w) v = __fmul_rn(v, nwv[j][b]);
          xv[j][b] = in ? v : 0.0f;
          if (in && blockIdx.x == 0 && a.xn_out) a.xn_out[k] = v;
        }
      }
    }
    if constexpr (XSRC != XS_PARTS) {
#pragma unroll
      for (int j = 0; j < NWT; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) g = fmaxf(g, fabsf(xv[j][b]));
    } else {
#pragma unroll
      for (int i = 0; i < kGpPerThread; ++i) g = fmaxf(g, __uint_as_float(gp[i]));
    }
    g = block_maxw<NW>(g, redf);
    const QuantDiv qd = make_qdiv(g);
    int rs = 0;
#pragma unroll
    for (int j = 0; j < NWT; ++j) {
      const int wd = tid + NT * j;
      if (wd < nw) {
        const uint32_t pk = quant_pack4(xv[j][0], xv[j][1], xv[j][2], xv[j][3], qd);
        rs = add_bytes(pk, rs);
        *reinterpret_cast<uint32_t*>(xq_lds + xslot(wd >> 2) + 4 * (wd & 3)) = pk;
        if (blockIdx.x == 0 && a.xq_out) reinterpret_cast<uint32_t*>(a.xq_out)[wd] = pk;
      }
    }
    rsum = block_sumw<NW>(rs, redi);  // its barrier also publishes xq_lds
    gx = g;
    if (blockIdx.x == 0 && tid == 0) {
      if (a.xs_out) a.xs_out[0] = g;
      if (a.rs_out) a.rs_out[0] = rsum;
    }
  }

  int part[R];
  gemv_dots<KC, R>(w, xq_lds, lane, C, part);
  float hmax = 0.0f;
  if (rb * RW < a.N) hmax = gemv_epilogue<R, EPI>(a, rb, part, rsum, gx, sw0, sw1);

  if constexpr (EPI == EPI_GATEUP) {
    __shared__ float redh[NW];
    hmax = block_maxw<NW>(hmax, redh);
    if (tid == 0) a.gh_parts[blockIdx.x] = hmax;
  }
}

// K beyond 4096 * 4 weights (int8 codes only): one row block per wave, K
// walked in segments of 16384 weights.
template <int R>
__global__ __launch_bounds__(256) void gemv_long_kernel(const GemvArgs a) {
  constexpr int KC = 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int C = (int)(a.Kp >> 6);
  const int wpr = (int)(a.Kp >> 4);
  const int64_t rb = (int64_t)blockIdx.x * 4 + wave;
  const int8_t* xq = reinterpret_cast<const int8_t*>(a.x);
  const float gx = a.x_scale[0];
  const int rsum = a.rowsum[0];
  int total[R];
#pragma unroll
  for (int r = 0; r < R; ++r) total[r] = 0;
  for (int seg = 0; seg < C; seg += 64 * KC) {
    uint4 w[R][KC];
    int x[KC][16];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int64_t n = rb * R + r;
      n = n < a.N ? n : a.N - 1;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        int c = seg + lane + 64 * i;
        c = c < C ? c : C - 1;
        w[r][i] = load_stream_u4(reinterpret_cast<const uint4*>(a.W0 + n * wpr) + c);
      }
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = seg + lane + 64 * i;
      const int cc = c < C ? c : C - 1;
      const int4* p = reinterpret_cast<const int4*>(xq + 64 * cc);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int4 v = p[q];
        if (c >= C) v = make_int4(0, 0, 0, 0);
        x[i][4 * q + 0] = v.x; x[i][4 * q + 1] = v.y; x[i][4 * q + 2] = v.z; x[i][4 * q + 3] = v.w;
      }
    }
    int part[R];
    gemv_dots_regs<KC, R>(w, x, part);
#pragma unroll
    for (int r = 0; r < R; ++r) total[r] += part[r];
  }
  if (rb * R < a.N) gemv_epilogue<R, EPI_STORE>(a, rb, total, rsum, gx, a.s0[0], 0.0f);
}

// ---------------------------------------------------------------------------
// Large layers (packed matrix of at least kPipeMinBytes): a streaming form.
// The grid is one block of 8 waves per CU; wave w walks the row blocks
// (2 rows each) w, w + T, w + 2T, ... (T = every wave of the grid), issuing
// the loads of its next row block before the dot products of the current
// one, so each wave keeps two row blocks (8 KiB at Kp = 8192) in flight for
// the whole launch instead of one burst per wave.  Every wave runs the same
// number of iterations, ceil(row blocks / T): rows past N are clamped on load
// and skipped on store, so the loop is uniform and the loads of one iteration
// are waited for one by one.
// The codes of this lane's chunks (lane, lane + 64) stay in registers for
// the whole launch.  Float activations are quantised once per block into LDS
// (the block's 512 threads share the row) and then taken into registers.
constexpr int kPipeWaves = 8;
constexpr int64_t kPipeMinBytes = 16ll << 20;

template <int KC, int R>
__device__ __forceinline__ void pipe_issue(const GemvArgs& a, int64_t rb, int lane, int C, int wpr,
                                           uint4 (&b)[R][KC]) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t n = rb * R + r;
    n = n < a.N ? n : a.N - 1;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      int c = lane + 64 * i;
      c = c < C ? c : C - 1;
      b[r][i] = load_stream_u4(reinterpret_cast<const uint4*>(a.W0 + n * wpr) + c);
    }
  }
}

template <int KC, int R>
__device__ __forceinline__ void pipe_rows(const GemvArgs& a, const uint4 (&b)[R][KC],
                                          const int (&x)[KC][16], int64_t rb, int rsum,
                                          float sc) {
  int part[R];
  gemv_dots_regs<KC, R>(b, x, part);
  const int lane = threadIdx.x & 63;
  const int sum = wave_transpose_reduce<R>(part);
  const int64_t n = rb * R + gemv_row<R>(lane);
  // rb past the last row block gives n >= N
  if (lane < R && n < a.N) {
    a.Y[n] = dequant(sum - rsum, sc);
    if (a.acc_out) a.acc_out[n] = sum - rsum;
  }
}

// IT > 0: exactly IT iterations, fully unrolled (straight-line code; for
// float input this measured 0.6 us faster on the 100B-class layer than the
// loop); IT == 0: the loop over pairs of iterations.
template <int KC, int XSRC, int IT>
__global__ __launch_bounds__(64 * kPipeWaves) void gemv_pipe_kernel(const GemvArgs a) {
  constexpr int R = 2, NW = kPipeWaves, NT = 64 * NW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gw = (int64_t)blockIdx.x * NW + wave;
  const int64_t T = (int64_t)gridDim.x * NW;
  const int C = (int)(a.Kp >> 6), wpr = (int)(a.Kp >> 4);
  const int64_t nrb = (a.N + R - 1) / R;
  uint4 bA[R][KC], bB[R][KC];
  int x[KC][16];
  int rsum;
  float gx;
  if constexpr (XSRC == XS_INT8) {
    const int8_t* xq = reinterpret_cast<const int8_t*>(a.x);
    int4 xv[KC][4];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = lane + 64 * i;
      const int4* p = reinterpret_cast<const int4*>(xq + 64 * (c < C ? c : C - 1));
#pragma unroll
      for (int q = 0; q < 4; ++q) xv[i][q] = p[q];
    }
    rsum = a.rowsum[0];
    gx = a.x_scale[0];
    pipe_issue<KC, R>(a, gw, lane, C, wpr, bA);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const bool ok = lane + 64 * i < C;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        x[i][4 * q + 0] = ok ? xv[i][q].x : 0;
        x[i][4 * q + 1] = ok ? xv[i][q].y : 0;
        x[i][4 * q + 2] = ok ? xv[i][q].z : 0;
        x[i][4 * q + 3] = ok ? xv[i][q].w : 0;
      }
    }
  } else {
    __shared__ __attribute__((aligned(16))) int8_t xl[4096 * KC];
    __shared__ float redf[NW];
    __shared__ int redi[NW];
    constexpr int NV = 4096 * KC / 4 / NT;  // groups of 4 values per thread
    const int K = (int)a.K, ng = (int)(a.Kp >> 2);
    const bool vec = (reinterpret_cast<uintptr_t>(a.x) & (XSRC == XS_BF16 ? 7 : 15)) == 0;
    float v[NV][4];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int g = tid + NT * j;
      if (vec && 4 * g + 3 < K) {
        if constexpr (XSRC == XS_BF16) {
          const uint2 u = reinterpret_cast<const uint2*>(a.x)[g];
          v[j][0] = __uint_as_float(u.x << 16);
          v[j][1] = __uint_as_float(u.x & 0xffff0000u);
          v[j][2] = __uint_as_float(u.y << 16);
          v[j][3] = __uint_as_float(u.y & 0xffff0000u);
        } else {
          const float4 f = reinterpret_cast<const float4*>(a.x)[g];
          v[j][0] = f.x; v[j][1] = f.y; v[j][2] = f.z; v[j][3] = f.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 4 * g + e;
          v[j][e] = (g < ng && k < K) ? load_act<XSRC == XS_BF16>(a.x, k) : 0.0f;
        }
      }
    }
    // float input: the first two row blocks go out before the quantisation
    pipe_issue<KC, R>(a, gw, lane, C, wpr, bA);
    if constexpr (IT > 1) pipe_issue<KC, R>(a, gw + T, lane, C, wpr, bB);
    __builtin_amdgcn_sched_barrier(0);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(v[j][e]));
    m = block_maxw<NW>(m, redf);
    const QuantDiv qd = make_qdiv(m);
    int rs = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int g = tid + NT * j;
      if (g < ng) {
        const uint32_t pk = quant_pack4(v[j][0], v[j][1], v[j][2], v[j][3], qd);
        rs = add_bytes(pk, rs);
        *reinterpret_cast<uint32_t*>(xl + 4 * g) = pk;
        if (blockIdx.x == 0 && a.xq_out) reinterpret_cast<uint32_t*>(a.xq_out)[g] = pk;
      }
    }
    rsum = block_sumw<NW>(rs, redi);  // its barrier also publishes xl
    gx = m;
    if (blockIdx.x == 0 && tid == 0) {
      if (a.xs_out) a.xs_out[0] = m;
      if (a.rs_out) a.rs_out[0] = rsum;
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
      const int c = lane + 64 * i;
      const bool ok = c < C;
      const int4* p = reinterpret_cast<const int4*>(xl + 64 * (ok ? c : 0));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int4 t = p[q];
        x[i][4 * q + 0] = ok ? t.x : 0;
        x[i][4 * q + 1] = ok ? t.y : 0;
        x[i][4 * q + 2] = ok ? t.z : 0;
        x[i][4 * q + 3] = ok ? t.w : 0;
      }
    }
  }
  const float sc = __fmul_rn(a.s0[0], gx);
  if constexpr (IT > 0) {
    // D row blocks in flight per wave: 3 for float input (the 100B-class
    // layer from fp32 11.6-11.8 -> 11.0-11.1 us), 2 for int8 codes (3 there
    // measured 0.1 us slower)
    constexpr int D = XSRC == XS_INT8 ? 2 : 3;
    uint4 bC[R][KC];
    uint4 (*buf[3])[KC] = {bA, bB, bC};
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      if (it + D - 1 < IT)
        pipe_issue<KC, R>(a, gw + (it + D - 1) * T, lane, C, wpr,
                          *reinterpret_cast<uint4(*)[R][KC]>(buf[(it + D - 1) % 3]));
      __builtin_amdgcn_sched_barrier(0);
      pipe_rows<KC, R>(a, *reinterpret_cast<uint4(*)[R][KC]>(buf[it % 3]), x, gw + it * T, rsum,
                       sc);
    }
    return;
  }
  // every wave runs the same number of iterations (grid-uniform); bA holds
  // iteration it on entry to each pair
  const int64_t ITr = (nrb + T - 1) / T;
  int64_t rb = gw;
  for (int64_t p = 0; p < (ITr - 1) / 2; ++p, rb += 2 * T) {
    pipe_issue<KC, R>(a, rb + T, lane, C, wpr, bB);
    __builtin_amdgcn_sched_barrier(0);
    pipe_rows<KC, R>(a, bA, x, rb, rsum, sc);
    pipe_issue<KC, R>(a, rb + 2 * T, lane, C, wpr, bA);
    __builtin_amdgcn_sched_barrier(0);
    pipe_rows<KC, R>(a, bB, x, rb + T, rsum, sc);
  }
  if ((ITr & 1) == 0) {  // two iterations left
    pipe_issue<KC, R>(a, rb + T, lane, C, wpr, bB);
    __builtin_amdgcn_sched_barrier(0);
    pipe_rows<KC, R>(a, bA, x, rb, rsum, sc);
    pipe_rows<KC, R>(a, bB, x, rb + T, rsum, sc);
  } else {
    pipe_rows<KC, R>(a, bA, x, rb, rsum, sc);
  }
}

// The streaming form for packed matrices of at least 16 MiB with Kp <= 8192.
static bool pipe_ok(int64_t K, int64_t N) {
  const int64_t Kp = (K + 63) / 64 * 64;
  return Kp <= 8192 && N * (Kp / 4) >= kPipeMinBytes;
}

template <int XSRC>
static hipError_t pipe_launch(const GemvArgs& a, hipStream_t s) {
  static int cus = 0;
  if (!cus) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
  }
  const dim3 grid((unsigned)cus), block(64 * kPipeWaves);
  const int64_t waves = (int64_t)cus * kPipeWaves, nrb = (a.N + 1) / 2;
  const int64_t it = (nrb + waves - 1) / waves;
#define BL_PIPE_IT(KCV)                                                                     \
  switch (it) {                                                                             \
    case 1: case 2: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 2>), grid, block, 0, s, a); break; \
    case 3: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 3>), grid, block, 0, s, a); break; \
    case 4: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 4>), grid, block, 0, s, a); break; \
    case 5: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 5>), grid, block, 0, s, a); break; \
    case 6: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 6>), grid, block, 0, s, a); break; \
    case 7: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 7>), grid, block, 0, s, a); break; \
    case 8: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 8>), grid, block, 0, s, a); break; \
    default: hipLaunchKernelGGL((gemv_pipe_kernel<KCV, XSRC, 0>), grid, block, 0, s, a); break; \
  }
  if (a.Kp <= 4096) {
    BL_PIPE_IT(1)
  } else {
    BL_PIPE_IT(2)
  }
#undef BL_PIPE_IT
  return hipGetLastError();
}

template <int R, int EPI, int XSRC, int NT = 256>
static hipError_t gemv_dispatch(GemvArgs a, hipStream_t s, int* nblocks = nullptr) {
  constexpr int RW = (EPI == EPI_GATEUP) ? R / 2 : R;
  const int64_t C = a.Kp / 64;
  const int64_t nrb = (a.N + RW - 1) / RW;
  if (C > 256) {
    if (XSRC != XS_INT8 || EPI != EPI_STORE) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemv_long_kernel<R>), dim3((unsigned)((nrb + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  constexpr int NW = NT / 64;
  const unsigned blocks = (unsigned)((nrb + NW - 1) / NW);
  if (nblocks) *nblocks = (int)blocks;
#define BL_GEMV_CASE(KCV) \
  hipLaunchKernelGGL((gemv_kernel<KCV, R, EPI, XSRC, NT>), dim3(blocks), dim3(NT), 0, s, a)
  if constexpr (XSRC == XS_NF32 || XSRC == XS_NBF16) {
    // the normalising prologue holds the row in registers: one chunk per lane
    // for the gate/up form (92 VGPRs; two chunks take 171), up to two for the
    // plain product
    if (C <= 64) {
      BL_GEMV_CASE(1);
      return hipGetLastError();
    }
    if constexpr (EPI == EPI_STORE) {
      if (C <= 128) {
        BL_GEMV_CASE(2);
        return hipGetLastError();
      }
    }
    return hipErrorInvalidValue;
  } else {
    if (C <= 64) BL_GEMV_CASE(1);
    else if (C <= 128) BL_GEMV_CASE(2);
    else if (C <= 192) BL_GEMV_CASE(3);
    else BL_GEMV_CASE(4);
    return hipGetLastError();
  }
#undef BL_GEMV_CASE
}

static GemvArgs base_args(int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y) {
  GemvArgs a = {};
  a.K = K;
  a.Kp = (K + 63) / 64 * 64;
  a.W0 = Wp;
  a.s0 = ws;
  a.N = N;
  a.Y = Y;
  return a;
}

constexpr int64_t kWideGemvBlocks = 192;  // 512-thread blocks at least this many

hipError_t launch_gemv(const int8_t* xq, const float* xs, const int32_t* rs, int64_t K,
                       const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                       int32_t* acc_out, hipStream_t s) {
  GemvArgs a = base_args(K, Wp, ws, N, Y);
  a.x = xq;
  a.x_scale = xs;
  a.rowsum = rs;
  a.acc_out = acc_out;
  if (pipe_ok(K, N)) return pipe_launch<XS_INT8>(a, s);
  // 2 rows per wave (measured against 4: 6912 -> 2560 3.31 -> 3.15 us,
  // 8192 -> 28672 11.65 -> 11.40 us)
  return gemv_dispatch<2, EPI_STORE, XS_INT8>(a, s);
}

// The one-burst fused kernels redo the row's quantisation in every block of
// 2 rows per wave; past ~7K inputs that redundant work costs more than a
// separate quantisation launch (8192 -> 28672: 15.5 us fused, 14.5 us for the
// quantiser and the int8 GEMV).  The streaming form quantises once per CU.
bool gemv_fused_ok(int64_t K, int64_t N) {
  return (K + 63) / 64 * 64 <= kFusedMaxKp || pipe_ok(K, N);
}

hipError_t launch_gemv_fused(const void* X, bool bf16, int64_t K, const uint32_t* Wp,
                             const float* ws, int64_t N, float* Y, int32_t* acc_out,
                             int8_t* xq_out, float* xs_out, int32_t* rs_out, hipStream_t s) {
  GemvArgs a = base_args(K, Wp, ws, N, Y);
  a.x = X;
  a.acc_out = acc_out;
  a.xq_out = xq_out;
  a.xs_out = xs_out;
  a.rs_out = rs_out;
  if (pipe_ok(K, N)) return bf16 ? pipe_launch<XS_BF16>(a, s) : pipe_launch<XS_F32>(a, s);
  // 8 waves per block halve the blocks that each redo the quantisation (2560
  // -> 6912: 3.98 -> 3.58 us); layers with fewer rows take 2 rows per wave
  // so that enough blocks remain (6912 -> 2560: 4.63 -> 3.85 us)
  if ((N + 31) / 32 >= kWideGemvBlocks)
    return bf16 ? gemv_dispatch<4, EPI_STORE, XS_BF16, 512>(a, s)
                : gemv_dispatch<4, EPI_STORE, XS_F32, 512>(a, s);
  return bf16 ? gemv_dispatch<2, EPI_STORE, XS_BF16, 512>(a, s)
              : gemv_dispatch<2, EPI_STORE, XS_F32, 512>(a, s);
}

hipError_t launch_gemv_parts(const float* X, const float* gparts, int nparts, int64_t K,
                             const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                             int8_t* xq_out, float* xs_out, int32_t* rs_out, hipStream_t s) {
  GemvArgs a = base_args(K, Wp, ws, N, Y);
  a.x = X;
  a.gparts = gparts;
  a.nparts = nparts;
  a.xq_out = xq_out;
  a.xs_out = xs_out;
  a.rs_out = rs_out;
  if ((N + 31) / 32 >= kWideGemvBlocks) return gemv_dispatch<4, EPI_STORE, XS_PARTS, 512>(a, s);
  return gemv_dispatch<2, EPI_STORE, XS_PARTS, 512>(a, s);
}

bool gemv_norm_ok(int64_t K) { return (K + 63) / 64 <= 128; }

hipError_t launch_gemv_norm(const float* X, int64_t K, const float* norm_w, float eps,
                            const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                            float* xn_out, int8_t* xq_out, float* xs_out, int32_t* rs_out,
                            hipStream_t s) {
  GemvArgs a = base_args(K, Wp, ws, N, Y);
  a.x = X;
  a.norm_w = norm_w;
  a.eps = eps;
  a.xn_out = xn_out;
  a.xq_out = xq_out;
  a.xs_out = xs_out;
  a.rs_out = rs_out;
  if ((N + 31) / 32 >= kWideGemvBlocks) return gemv_dispatch<4, EPI_STORE, XS_NF32, 512>(a, s);
  return gemv_dispatch<2, EPI_STORE, XS_NF32, 512>(a, s);
}

constexpr int kGateupR = 4;  // weight rows per wave in the gate/up GEMV (half gate, half up)

// the gate/up epilogue exists in the one-pass kernel only (K up to 4096 * 4)
bool gemv_gateup_ok(int64_t K) { return (K + 63) / 64 <= 256; }

// one partial maximum per block: 4 waves x kGateupR/2 output rows
int64_t gemv_gateup_parts(int64_t N) { return (N + 2 * kGateupR - 1) / (2 * kGateupR); }

bool gemv_gateup_norm_ok(int64_t K) { return (K + 63) / 64 <= 64; }

hipError_t launch_gemv_gateup_norm(const void* H, bool bf16, int64_t K, const float* norm_w,
                                   float eps, const uint32_t* Wg, const float* sg,
                                   const uint32_t* Wu, const float* su, int64_t N, float* Hout,
                                   float* gh_parts, int* nparts, float* xn_out, int8_t* xq_out,
                                   float* xs_out, int32_t* rs_out, hipStream_t s) {
  GemvArgs a = base_args(K, Wg, sg, N, Hout);
  a.x = H;
  a.W1 = Wu;
  a.s1 = su;
  a.gh_parts = gh_parts;
  a.norm_w = norm_w;
  a.eps = eps;
  a.xn_out = xn_out;
  a.xq_out = xq_out;
  a.xs_out = xs_out;
  a.rs_out = rs_out;
  // 8-wave blocks: half as many blocks redo the norm as with 4
  return bf16 ? gemv_dispatch<kGateupR, EPI_GATEUP, XS_NBF16, 512>(a, s, nparts)
              : gemv_dispatch<kGateupR, EPI_GATEUP, XS_NF32, 512>(a, s, nparts);
}

hipError_t launch_gemv_gateup(const int8_t* xq, const float* xs, const int32_t* rs, int64_t K,
                              const uint32_t* Wg, const float* sg, const uint32_t* Wu,
                              const float* su, int64_t N, float* H, float* gh_parts,
                              int* nparts, hipStream_t s) {
  GemvArgs a = base_args(K, Wg, sg, N, H);
  a.x = xq;
  a.x_scale = xs;
  a.rowsum = rs;
  a.W1 = Wu;
  a.s1 = su;
  a.gh_parts = gh_parts;
  *nparts = (int)gemv_gateup_parts(N);
  return gemv_dispatch<kGateupR, EPI_GATEUP, XS_INT8>(a, s);
}

}  // namespace bl

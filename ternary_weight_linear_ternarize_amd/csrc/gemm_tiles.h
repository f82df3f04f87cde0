// Tiled ternary x int8 GEMM kernel (v_mfma_i32_32x32x32_i8) for M > 64.
#pragma once

#include "bl_device.h"

namespace bl {

__device__ __forceinline__ uint32_t pick32(const u32x4& v, int s) {
  return s == 0 ? v[0] : s == 1 ? v[1] : s == 2 ? v[2] : v[3];
}

// ((float)a * s) / 127 with one rounding per operation, as dequant(), computed
// as RN32(RN64(p * RN64(1/127))) with p = RN32(a * s).  This is exact: p has
// at most 24 significant bits, so p / 127 differs from every binary32 rounding
// midpoint by at least 2^-25 / 127 of its magnitude (127 is odd, a midpoint
// has 25 bits), far more than the 2^-52 relative error of the binary64
// product.  Holds for subnormal quotients too (binary64 keeps them normal).
__device__ __forceinline__ float dequant_f64(int a, float s) {
  const float p = __fmul_rn((float)a, s);
  return (float)((double)p * (1.0 / 127.0));
}

// ---------------------------------------------------------------------------
// Block tile BM x BN = (32 TM WAVES_M) x (32 TN WAVES_N), 4 waves, wave tile
// (32 TM) x (32 TN).  K advances in chunks of 256 (10 for K = 2560):
//
//  * activations: BM x 256 int8 per chunk go HBM/L2 -> LDS directly
//    (buffer_load ... lds, 64 lanes x 16 bytes per load = 4 rows x 256 bytes),
//    double buffered.  Each load writes 1 KB of LDS in lane order; the lane
//    that lands in 16-byte slot t of row r fetches logical piece t ^ (r % 16),
//    so a wave reading piece p of 32 consecutive rows hits 16 distinct bank
//    groups (conflict-free ds_read_b128) while every load still covers whole
//    256-byte row segments of global memory.
//  * packed weights go straight to registers (buffer loads, double buffered
//    across chunks): lane (li, g) of 32-row tile tn holds words 8g .. 8g+7 of
//    the chunk for weight row 32 tn + li.
//
// MFMA operands: in k-step s of a chunk, lane (li, g) supplies activation
// bytes 16 (8g + s) .. +15 of token row li and the four code vectors of
// packed word 8g + s of weight row li; both cover the same 16 k positions, and
// the MFMA sums over all k of the step whatever their order among lanes.
//
// The accumulators start at -rowsum (per token row), so they end as
// sum q (t + 1) - sum q = sum q t.  Result layout of one 32x32 tile (lane l,
// g = l / 32, register r): token row 8 (r / 4) + 4 g + (r % 4), weight row
// l % 32.  The epilogue of an interior tile dequantises in registers, writes
// the tile to LDS row-major (the activation buffers are free by then) in
// passes of as many rows as fit, and stores whole 1 KB row segments, 16
// bytes per lane (non-temporal: Y is not read back here); against one
// 4-byte store per register (two 128-byte row segments) this takes 37-38 us
// instead of 42-43 for 2048 x 2560 x 6912.  Edge tiles, tiles narrower than
// 256 columns, and calls that also want the int32 accumulators store from
// the registers directly.
//
// Out-of-range rows and the K tail read as zero through the buffer
// resources' bounds, so the main loop has no per-lane range checks.  Block b
// runs on XCD b % 8; bm varies fastest so the blocks one XCD runs share
// activation rows in its L2.
//
// NB = 2 (the FFN's gate/up): the block's BN columns of both weight
// matrices, h = relu(gate)^2 * up in the epilogue (from the registers), and
// the block's max |h| per token row in gh_parts[bn M + m].
template <int TM, int TN, int WAVES_M, int WAVES_N, int NB = 1>
struct TiledGemm {
  static constexpr int KCH = 256;
  static constexpr int BM = 32 * TM * WAVES_M, BN = 32 * TN * WAVES_N;
  static constexpr int ABYTES = BM * KCH;  // one LDS stage of activations
  static constexpr int NLD = BM / 16;      // direct loads per wave per chunk
  static constexpr int LDS = 2 * ABYTES + 8 * BM + (NB == 2 ? 8 * BM : 0);
};

template <int TM, int TN, int WAVES_M, int WAVES_N, int MINB = 2, int NB = 1>
__global__ __launch_bounds__(256, MINB) void tiled_gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int64_t M, int64_t Kp, const uint32_t* __restrict__ W,
    const float* __restrict__ w_scale, int64_t N, float* __restrict__ Y,
    int32_t* __restrict__ acc_out, int nbm, const uint32_t* __restrict__ W1 = nullptr,
    const float* __restrict__ w1_scale = nullptr, float* __restrict__ gh_parts = nullptr) {
  using G = TiledGemm<TM, TN, WAVES_M, WAVES_N, NB>;
  constexpr int KCH = G::KCH, BM = G::BM, BN = G::BN, ABYTES = G::ABYTES, NLD = G::NLD;
  constexpr int WPL = KCH / 32;  // k-steps per chunk
  constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource
  static_assert(WAVES_M * WAVES_N == 4, "4 waves per block");
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  float* lds_sc = reinterpret_cast<float*>(lds + 2 * ABYTES);
  int32_t* lds_rs = reinterpret_cast<int32_t*>(lds + 2 * ABYTES + 4 * BM);
  float* lds_sc1 = reinterpret_cast<float*>(lds + 2 * ABYTES + 8 * BM);         // NB == 2
  uint32_t* lds_hm = reinterpret_cast<uint32_t*>(lds + 2 * ABYTES + 12 * BM);  // NB == 2

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int g = lane >> 5, li = lane & 31;
  // block-uniform by construction; readfirstlane lets the compiler see it, so
  // the buffer resources stay in SGPRs (otherwise every buffer load is
  // wrapped in a loop over distinct resource values)
  const int bm = __builtin_amdgcn_readfirstlane(blockIdx.x % nbm);
  const int bn = __builtin_amdgcn_readfirstlane(blockIdx.x / nbm);
  const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;
  const int64_t wpr = Kp / 16;
  const int nchunks = (int)((Kp + KCH - 1) / KCH);
  const int mrows = __builtin_amdgcn_readfirstlane((int)(M - m0 < BM ? M - m0 : BM));
  const int nrows = __builtin_amdgcn_readfirstlane((int)(N - n0 < BN ? N - n0 : BN));
  const buf_rsrc ra = make_buf_rsrc(Xq + m0 * Kp, (uint32_t)(mrows * Kp));
  const buf_rsrc rb = make_buf_rsrc(W + n0 * wpr, (uint32_t)(nrows * wpr * 4));
  const buf_rsrc rb1 = make_buf_rsrc((NB == 2 ? W1 : W) + n0 * wpr, (uint32_t)(nrows * wpr * 4));

  // activation loads: load j of this wave fills rows 4 (wave NLD + j) + lane / 16
  uint32_t a_off[NLD];
  int a_pl[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int row = 4 * (wave * NLD + j) + (lane >> 4);
    a_pl[j] = (lane & 15) ^ (row & 15);
    a_off[j] = (uint32_t)(row * Kp + 16 * a_pl[j]);
  }
  // 32-bit range tests (K is far below 2^31): piece j of this lane is in
  // range while kc < a_lim[j]
  int a_lim[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) a_lim[j] = (int)Kp - 16 * a_pl[j];
  auto issue_a = [&](int c, int buf) {
    const int kc = c * KCH;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      const uint32_t off = kc < a_lim[j] ? a_off[j] + (uint32_t)kc : kOOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds + buf * ABYTES + (wave * NLD + j) * 1024, 16,
                                               off, 0, 0, 0);
    }
  };
  uint32_t b_off[TN];
#pragma unroll
  for (int tn = 0; tn < TN; ++tn)
    b_off[tn] = (uint32_t)(((32 * (wn * TN + tn) + li) * wpr + 8 * g) * 4);
  const int b_lim = (int)wpr - 8 * g;  // words w0 + 4q + (0..3) in range while w0 + 4q < b_lim
  auto issue_b = [&](int c, u32x4 (&dst)[NB][TN][2]) {
    const int w0 = c * (KCH / 16);
#pragma unroll
    for (int mat = 0; mat < NB; ++mat)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t off =
              w0 + 4 * q < b_lim ? b_off[tn] + (uint32_t)((w0 + 4 * q) * 4) : kOOB;
          dst[mat][tn][q] = __builtin_amdgcn_raw_buffer_load_b128(mat == 0 ? rb : rb1, off, 0, 0);
        }
  };
  // LDS byte offset of the activation operand of k-step s (tile tm adds 32 tm rows)
  uint32_t a_rd[WPL];
#pragma unroll
  for (int s = 0; s < WPL; ++s)
    a_rd[s] = (uint32_t)((32 * wm * TM + li) * KCH + 16 * ((8 * g + s) ^ (li & 15)));

  u32x4 bA[NB][TN][2], bB[NB][TN][2];
  issue_a(0, 0);
  issue_b(0, bA);
  {
    const float sw = w_scale[0];
    const float sw1 = NB == 2 ? w1_scale[0] : 0.0f;
    for (int i = tid; i < BM; i += 256) {
      const int64_t m = m0 + i;
      lds_sc[i] = m < M ? __fmul_rn(sw, x_scale[m]) : 0.0f;
      lds_rs[i] = m < M ? rowsum[m] : 0;
      if constexpr (NB == 2) {
        lds_sc1[i] = m < M ? __fmul_rn(sw1, x_scale[m]) : 0.0f;
        lds_hm[i] = 0u;
      }
    }
  }
  __syncthreads();
  v16i acc[NB][TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int v = -lds_rs[32 * (wm * TM + tm) + 8 * (r >> 2) + 4 * g + (r & 3)];
#pragma unroll
      for (int mat = 0; mat < NB; ++mat)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[mat][tm][tn][r] = v;
    }

  auto compute = [&](int buf, const u32x4 (&b)[NB][TN][2]) {
    const int8_t* base = lds + buf * ABYTES;
    v4i a[2][TM];
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
      a[0][tm] = *reinterpret_cast<const v4i*>(base + a_rd[0] + tm * 32 * KCH);
#pragma unroll
    for (int s = 0; s < WPL; ++s) {
      if (s + 1 < WPL) {
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          a[(s + 1) & 1][tm] = *reinterpret_cast<const v4i*>(base + a_rd[s + 1] + tm * 32 * KCH);
      }
#pragma unroll
      for (int mat = 0; mat < NB; ++mat)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const v4i bv = codes_operand(pick32(b[mat][tn][s >> 2], s & 3));
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
            acc[mat][tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[s & 1][tm], bv,
                                                                    acc[mat][tm][tn], 0, 0, 0);
        }
    }
  };
  // Chunk c: wait for its loads (issued one chunk earlier), then start chunk
  // c + 1's loads into the other buffers and compute.  The barrier also
  // guarantees every wave has finished reading the buffer about to be refilled.
  auto step = [&](int c, int buf, const u32x4 (&cur)[NB][TN][2], u32x4 (&nxt)[NB][TN][2]) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c + 1 < nchunks) {
      issue_a(c + 1, buf ^ 1);
      issue_b(c + 1, nxt);
    }
    compute(buf, cur);
  };
  for (int c = 0; c < nchunks; c += 2) {
    step(c, 0, bA, bB);
    if (c + 1 < nchunks) step(c + 1, 1, bB, bA);
  }

  if constexpr (NB == 2) {
    // h = relu(gate)^2 * up per element, and max |h| per token row: over the
    // 32 lanes of a column group, then the waves through LDS
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = 32 * (wm * TM + tm) + 8 * (r >> 2) + 4 * g + (r & 3);
        const float scg = lds_sc[ml], scu = lds_sc1[ml];
        float hm = 0.0f;
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int nl = 32 * (wn * TN + tn) + li;
          if (ml < mrows && nl < nrows) {
            const float gv = dequant_f64(acc[0][tm][tn][r], scg);
            const float uv = dequant_f64(acc[NB - 1][tm][tn][r], scu);
            const float rl = gv > 0.0f ? gv : 0.0f;
            const float hv = __fmul_rn(__fmul_rn(rl, rl), uv);
            Y[(m0 + ml) * N + n0 + nl] = hv;
            hm = fmaxf(hm, fabsf(hv));
          }
        }
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) hm = fmaxf(hm, __shfl_xor(hm, o));
        if (li == 0 && hm > 0.0f) atomicMax(&lds_hm[ml], __float_as_uint(hm));
      }
    }
    __syncthreads();
    for (int i = tid; i < mrows; i += 256)
      gh_parts[(int64_t)bn * M + m0 + i] = __uint_as_float(lds_hm[i]);
    return;
  } else if (BN % 256 == 0 && mrows == BM && nrows == BN && !acc_out) {
    // RP rows of the tile per pass through the two activation buffers
    constexpr int RP = (2 * ABYTES) / (BN * 4) >= BM ? BM : BM / 2;
    static_assert(RP * BN * 4 <= 2 * ABYTES && BM % RP == 0 && RP % 32 == 0 && RP % 4 == 0,
                  "epilogue passes");
    constexpr int SEG = BN / 256 > 0 ? BN / 256 : 1;  // 1 KB segments per row
    float* ep = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int p = 0; p < BM / RP; ++p) {
      __syncthreads();  // the buffers are no longer read (first pass) or stored (later passes)
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int rt = 32 * (wm * TM + tm);
        if (rt >= p * RP && rt < (p + 1) * RP) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ml = rt + 8 * (r >> 2) + 4 * g + (r & 3);
            const float sc = lds_sc[ml];
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
              ep[(ml - p * RP) * BN + 32 * (wn * TN + tn) + li] = dequant_f64(acc[0][tm][tn][r], sc);
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < RP * SEG / 4; ++j) {
        const int u = wave * (RP * SEG / 4) + j;  // segment u of the pass
        const int rl = u / SEG, col = (u % SEG) * 256 + 4 * lane;
        const f32x4 v = *reinterpret_cast<const f32x4*>(ep + rl * BN + col);
        __builtin_nontemporal_store(
            v, reinterpret_cast<f32x4*>(Y + (m0 + p * RP + rl) * N + n0 + col));
      }
    }
    return;
  }
  // Edge tiles and accumulator output: straight from the registers.
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ml = 32 * (wm * TM + tm) + 8 * (r >> 2) + 4 * g + (r & 3);
      const float sc = lds_sc[ml];
      float* yrow = Y + (m0 + ml) * N + n0 + 32 * wn * TN + li;
      if (ml < mrows) {
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int nl = 32 * (wn * TN + tn) + li;
          if (nl < nrows) {
            __builtin_nontemporal_store(dequant_f64(acc[0][tm][tn][r], sc), yrow + 32 * tn);
            if (acc_out) acc_out[(m0 + ml) * N + n0 + nl] = acc[0][tm][tn][r];
          }
        }
      }
    }
  }
}

}  // namespace bl

// Tiled ternary x int8 GEMM kernel template (v_mfma_i32_32x32x32_i8).
#pragma once

#include "bl_device.h"

namespace bl {

__device__ __forceinline__ v4i unpack_operand32(uint32_t w) {
  v4i r;
  r[0] = (int)(w & 0x03030303u);
  r[1] = (int)((w >> 2) & 0x03030303u);
  r[2] = (int)((w >> 4) & 0x03030303u);
  r[3] = (int)((w >> 6) & 0x03030303u);
  return r;
}

__device__ __forceinline__ uint32_t pick32(const uint4& v, int s) {
  return s == 0 ? v.x : s == 1 ? v.y : s == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Prefill GEMM on v_mfma_i32_32x32x32_i8.
//
// Block tile BM x BN, 4 waves as WAVES_M x WAVES_N, wave tile (32 TM) x (32 TN).
// K advances in chunks of KCH: the activation chunk (BM x KCH int8) is staged
// through LDS (double buffered, rows padded by 16 bytes so the 32 rows a wave
// reads at one offset spread over the banks); the packed weight chunk goes
// straight to registers (KCH/32 words per lane per 32-row tile).  Loads of
// chunk c+1 are issued before chunk c is computed.
//
// Result layout of one 32x32 tile (lane l, g = l / 32, register r):
// token row 8 (r / 4) + 4 g + (r % 4), weight row l % 32.
//
// Blocks are numbered so that block b runs on XCD b % 8; the M tiles are
// spread over XCDs (bm varies fastest within a round of 8) so the blocks one
// XCD runs share activation rows in that XCD's L2.

// KCH: K per chunk (a multiple of 64); lane group g holds words
// (KCH/32) g .. (KCH/32) g + KCH/32 - 1 of each chunk row, and k-step s
// (0 <= s < KCH/32) uses word (KCH/32) g + s with the activation bytes at
// 16 ((KCH/32) g + s).
template <int TM, int TN, int WAVES_M, int WAVES_N, int KCH>
__global__ __launch_bounds__(256, 2) void mfma32_gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int64_t M, int64_t Kp, const uint32_t* __restrict__ W,
    const float* __restrict__ w_scale, int64_t N, float* __restrict__ Y,
    int32_t* __restrict__ acc_out, int nbm, int nbn) {
  static_assert(WAVES_M * WAVES_N == 4, "4 waves per block");
  constexpr int BM = 32 * TM * WAVES_M;
  constexpr int BN = 32 * TN * WAVES_N;
  constexpr int PITCH = KCH + 16;             // padded row: spreads a column over all banks
  constexpr int CPR = KCH / 16;               // 16-byte pieces per row per chunk
  constexpr int A_U4 = BM * CPR / 256;        // uint4 per thread per chunk
  constexpr int WPL = KCH / 32;               // words per lane per chunk = k-steps
  constexpr int BU4 = WPL / 4;                // uint4 per lane per 32-row tile
  static_assert(A_U4 >= 1 && WPL % 4 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) int8_t lds_a[2][BM * PITCH];
  __shared__ float lds_sc[BM];    // g_w * g_x per token row of the tile
  __shared__ int32_t lds_rs[BM];  // row sums of the codes

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int g = lane >> 5, li = lane & 31;
  // block -> tile: bm fastest, so the blocks of one XCD (b % 8) share A rows
  const int bm = blockIdx.x % nbm, bn = blockIdx.x / nbm;
  const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;
  const int64_t wpr = Kp / 16;
  const int nchunks = (int)((Kp + KCH - 1) / KCH);

  uint4 a_reg[A_U4];
  auto load_a = [&](int64_t kc) {
#pragma unroll
    for (int i = 0; i < A_U4; ++i) {
      const int u = tid + 256 * i;
      const int row = u / CPR, c16 = u % CPR;
      const int64_t m = m0 + row, k = kc + 16 * c16;
      if (m < M && k < Kp)
        a_reg[i] = *reinterpret_cast<const uint4*>(Xq + m * Kp + k);
      else
        a_reg[i] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_U4; ++i) {
      const int u = tid + 256 * i;
      const int row = u / CPR, c16 = u % CPR;
      *reinterpret_cast<uint4*>(&lds_a[buf][row * PITCH + 16 * c16]) = a_reg[i];
    }
  };
  uint4 b_reg[TN][BU4];
  auto load_b = [&](int64_t kc) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int64_t n = n0 + 32 * (wn * TN + tn) + li;
#pragma unroll
      for (int q = 0; q < BU4; ++q) {
        const int64_t word = kc / 16 + WPL * g + 4 * q;
        if (n < N && word < wpr)
          b_reg[tn][q] = *reinterpret_cast<const uint4*>(W + n * wpr + word);
        else
          b_reg[tn][q] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };

  v16i acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tm][tn][r] = 0;

  load_a(0);
  load_b(0);
  {
    const float sw = w_scale[0];
    for (int i = tid; i < BM; i += 256) {
      const int64_t m = m0 + i;
      lds_sc[i] = m < M ? __fmul_rn(sw, x_scale[m]) : 0.0f;
      lds_rs[i] = m < M ? rowsum[m] : 0;
    }
  }
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    store_a(buf);
    uint4 b_cur[TN][BU4];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int q = 0; q < BU4; ++q) b_cur[tn][q] = b_reg[tn][q];
    __syncthreads();
    if (c + 1 < nchunks) {
      load_a((int64_t)(c + 1) * KCH);
      load_b((int64_t)(c + 1) * KCH);
    }
    const int8_t* la = &lds_a[buf][0];
#pragma unroll
    for (int s = 0; s < WPL; ++s) {
      v4i a[TM];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
        const int row = 32 * (wm * TM + tm) + li;
        a[tm] = *reinterpret_cast<const v4i*>(la + row * PITCH + 16 * (WPL * g + s));
      }
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const v4i b = unpack_operand32(pick32(b_cur[tn][s >> 2], s & 3));
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
          acc[tm][tn] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[tm], b, acc[tm][tn], 0, 0, 0);
      }
    }
  }

  // Epilogue: dequantise one 32x32 tile at a time into a wave-private LDS
  // patch, then write whole 16-byte runs of Y rows (non-temporal: Y is
  // written once and not read back here).
  constexpr int OP = 36;  // floats per staged row (32 + 4 pad)
  static_assert(4 * 32 * OP * 4 <= 2 * BM * PITCH, "staging fits in the A buffers");
  __syncthreads();
  float* st = reinterpret_cast<float*>(&lds_a[0][0]) + wave * 32 * OP;
  const bool vec = (N & 3) == 0 && (reinterpret_cast<uintptr_t>(Y) & 15) == 0;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rl = 8 * (r >> 2) + 4 * g + (r & 3);
        const int ml = 32 * (wm * TM + tm) + rl;
        const int a = acc[tm][tn][r] - lds_rs[ml];
        st[rl * OP + li] = dequant_fast(a, lds_sc[ml]);
        if (acc_out) {
          const int64_t m = m0 + ml, n = n0 + 32 * (wn * TN + tn) + li;
          if (m < M && n < N) acc_out[m * N + n] = a;
        }
      }
      // the patch is private to this wave: a wave-level barrier orders it
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int idx = lane + 64 * j;  // float4 index in the 32 x 32 patch
        const int rl = idx >> 3, c4 = idx & 7;
        const int64_t m = m0 + 32 * (wm * TM + tm) + rl;
        const int64_t n = n0 + 32 * (wn * TN + tn) + 4 * c4;
        if (m >= M) continue;
        const float* src = st + rl * OP + 4 * c4;
        if (vec && n + 3 < N) {
          f32x4 v = {src[0], src[1], src[2], src[3]};
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(Y + m * N + n));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < N) Y[m * N + n + e] = src[e];
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

}  // namespace bl

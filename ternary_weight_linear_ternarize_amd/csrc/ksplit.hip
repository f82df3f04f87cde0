// Ternary x int8 product for 2..384 tokens with K split over every wave of
// the block and every load of a wave issued before the first MFMA.
//
// youngju.dev "BitNet論文分析", section "BitNet b1.58": the integer product is
// F.linear(x_q, w_q) followed by output * (w_scale * x_scale) / Q; here in
// the shifted-code form acc = sum_k q[m][k] * (t[n][k] + 1) - rowsum[m] on
// v_mfma_i32_16x16x64_i8 (dashen-tech "BitNet.cpp 深度解析" §3.1: the
// product equals sum_pos - sum_neg).
//
// At these token counts a layer moves a few MB (the 2B-class FFN at 64
// tokens: 8.8 MB of gate/up weights, 160 KB of activation codes), so its time
// is set by how many bytes each CU has in flight, not by the matrix cores;
// chains of dependent K chunks (one per 256 weights in the block-tile and
// tiled kernels) are what it removes.
// A block owns a BM x BN output tile (BM = 16 TM tokens, BN = 16 TN columns
// of each of NB weight matrices) and its W waves split K between them: K is
// cut into pieces of 256, wave w takes pieces [w ppw, (w + 1) ppw), and all
// of them -- activation rows and weight words -- are loaded into registers
// at once, as branch-free buffer loads (rows past M or N and pieces past Kp
// read zero).  The MFMAs of piece j then wait only for piece j's loads.  The
// W partial tiles are added through LDS and the block's threads share the
// epilogue.
//
// Operand mapping, lane l = 16 g + li: in piece h, lane group g owns weights
// 256 h + 64 g .. +63, i.e. packed words 16 h + 4 g .. +3 of a row (word j
// holds weights 16 j .. 16 j + 15, codes_operand unpacks them in order), one
// 16-byte load per row, so a load instruction reads 64 contiguous bytes of
// each of 16 rows (pieces of 128 weights, 8-byte loads and 32-byte runs,
// measured 0.1-1.4 us slower on every shape this kernel runs); step s (0..3)
// feeds word 16 h + 4 g + s of column row li and the 16 activation bytes at
// 256 h + 64 g + 16 s of token row li.  Result lane l, register r holds
// (token 4 g + r, column li).
#include "bl_device.h"
#include "bl_launch.h"

namespace bl {

enum { KS_STORE = 0, KS_GATEUP = 1 };

constexpr int kPiece = 256;  // K per piece

template <int NB, int TM, int TN, int W, int CPW, int EPI>
__global__ __launch_bounds__(64 * W) void mfma_ksplit_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int64_t M, int64_t Kp,
    const uint32_t* __restrict__ W0, const float* __restrict__ s0,
    const uint32_t* __restrict__ W1, const float* __restrict__ s1, int64_t N,
    float* __restrict__ Y, int32_t* __restrict__ acc_out, float* __restrict__ gh_parts, int nbn,
    int ppw) {
  constexpr int BM = 16 * TM, BN = 16 * TN;
  constexpr int J = NB * TM * TN;  // accumulator tiles per wave
  constexpr int NT = 64 * W;
  extern __shared__ __attribute__((aligned(16))) v4i ks_lds[];
  v4i* part = ks_lds;                                              // [W][J][64]
  float* tokx = reinterpret_cast<float*>(ks_lds + W * J * 64);     // [BM]
  int* tokr = reinterpret_cast<int*>(tokx + BM);                   // [BM]
  uint32_t* hred = reinterpret_cast<uint32_t*>(tokr + BM);         // [BM]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int bid = __builtin_amdgcn_readfirstlane(blockIdx.x);
  const int bn = bid % nbn, bm = bid / nbn;
  const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;
  const int64_t wpr = Kp / 16;
  const int64_t npieces = (Kp + kPiece - 1) / kPiece;
  const int64_t h0 = (int64_t)wave * ppw;
  const int64_t hn = npieces - h0 < ppw ? npieces - h0 : ppw;  // pieces of this wave (may be <= 0)

  // the epilogue's per-token operands, early (tokens past M read 0)
  float tx = 0.0f;
  int tr = 0;
  if (tid < BM) {
    const buf_rsrc rx = make_buf_rsrc(x_scale, (uint32_t)(4 * M));
    const buf_rsrc rr = make_buf_rsrc(rowsum, (uint32_t)(4 * M));
    const uint32_t off = m0 + tid < M ? (uint32_t)(4 * (m0 + tid)) : 0x80000000u;
    tx = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0));
    tr = (int)__builtin_amdgcn_raw_buffer_load_b32(rr, off, 0, 0);
  }
  const float ws0 = s0[0], ws1 = NB == 2 ? s1[0] : 0.0f;

  const int64_t mrows = M - m0 < BM ? M - m0 : BM;
  const int64_t nrows = N - n0 < BN ? N - n0 : BN;
  const buf_rsrc ra = make_buf_rsrc(Xq + m0 * Kp, (uint32_t)(mrows * Kp));
  const buf_rsrc rb0 = make_buf_rsrc(W0 + n0 * wpr, (uint32_t)(nrows * wpr * 4));
  const buf_rsrc rb1 = make_buf_rsrc((NB == 2 ? W1 : W0) + n0 * wpr, (uint32_t)(nrows * wpr * 4));

  // ---- every load of the wave, piece by piece
  constexpr int NS = kPiece / 64;  // MFMA k-steps per piece
  u32x4 a_reg[CPW][TM][NS];
  u32x4 b_reg[CPW][NB][TN];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int64_t h = h0 + j;
    const bool live = j < hn;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int64_t k = kPiece * h + 16 * NS * g + 16 * s;
        const uint32_t off =
            live && k < Kp ? (uint32_t)((16 * tm + li) * Kp + k) : 0x80000000u;
        a_reg[j][tm][s] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
      }
    }
    const int64_t word = (kPiece / 16) * h + NS * g;
#pragma unroll
    for (int mat = 0; mat < NB; ++mat) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        const uint32_t off = live && word < wpr
                                 ? (uint32_t)(((16 * tn + li) * wpr + word) * 4)
                                 : 0x80000000u;
        b_reg[j][mat][tn] = __builtin_amdgcn_raw_buffer_load_b128(mat == 0 ? rb0 : rb1, off, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  v4i acc[NB][TM][TN];
#pragma unroll
  for (int mat = 0; mat < NB; ++mat)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[mat][tm][tn] = v4i{0, 0, 0, 0};

#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    if (j < hn) {  // uniform over the wave
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int mat = 0; mat < NB; ++mat) {
#pragma unroll
          for (int tn = 0; tn < TN; ++tn) {
            const v4i b = codes_operand(b_reg[j][mat][tn][s]);
#pragma unroll
            for (int tm = 0; tm < TM; ++tm)
              acc[mat][tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                  __builtin_bit_cast(v4i, a_reg[j][tm][s]), b, acc[mat][tm][tn], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- the W partial tiles meet in LDS
#pragma unroll
  for (int mat = 0; mat < NB; ++mat)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        part[(wave * J + (mat * TM + tm) * TN + tn) * 64 + lane] = acc[mat][tm][tn];
  if (tid < BM) {
    tokx[tid] = tx;
    tokr[tid] = tr;
    hred[tid] = 0u;
  }
  __syncthreads();

  // ---- epilogue: slot = (tm, tn, lane) of the tile, all NB matrices
  constexpr int SLOTS = TM * TN * 64;
  for (int slot = tid; slot < SLOTS; slot += NT) {  // the same trip count for a whole wave
    const int sl = slot & 63, jt = slot >> 6;
    const int tm = jt / TN, tn = jt % TN;
    const int sg = sl >> 4, sli = sl & 15;
    v4i sum[NB];
#pragma unroll
    for (int mat = 0; mat < NB; ++mat) {
      v4i t = part[((mat * TM + tm) * TN + tn) * 64 + sl];
#pragma unroll
      for (int w = 1; w < W; ++w) t += part[(w * J + (mat * TM + tm) * TN + tn) * 64 + sl];
      sum[mat] = t;
    }
    const int64_t n = n0 + 16 * tn + sli;
    if constexpr (EPI == KS_STORE) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = 16 * tm + 4 * sg + r;
        const int64_t m = m0 + lrow;
        if (m < M && n < N) {
          const int a = sum[0][r] - tokr[lrow];
          if (Y) Y[m * N + n] = dequant_fast(a, __fmul_rn(ws0, tokx[lrow]));
          if (acc_out) acc_out[m * N + n] = a;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = 16 * tm + 4 * sg + r;
        const int64_t m = m0 + lrow;
        float hm = 0.0f;
        if (m < M && n < N) {
          const int rsm = tokr[lrow];
          const float xs = tokx[lrow];
          const float gv = dequant_fast(sum[0][r] - rsm, __fmul_rn(ws0, xs));
          const float uv = dequant_fast(sum[1][r] - rsm, __fmul_rn(ws1, xs));
          const float rl = gv > 0.0f ? gv : 0.0f;
          const float hv = __fmul_rn(__fmul_rn(rl, rl), uv);
          Y[m * N + n] = hv;
          hm = fabsf(hv);
          hm = hm == hm ? hm : 0.0f;  // a NaN h does not enter the maximum
        }
        // max over the 16 lanes holding this token row
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) hm = fmaxf(hm, __shfl_xor(hm, o));
        if (sli == 0 && hm > 0.0f) atomicMax(&hred[lrow], __float_as_uint(hm));
      }
    }
  }
  if constexpr (EPI == KS_GATEUP) {
    __syncthreads();
    if (tid < BM && m0 + tid < M) gh_parts[(int64_t)bn * M + m0 + tid] = __uint_as_float(hred[tid]);
  }
}

template <int NB, int TM, int TN, int W, int CPW, int EPI>
static hipError_t ksplit_go(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                            int64_t Kp, const uint32_t* W0, const float* s0, const uint32_t* W1,
                            const float* s1, int64_t N, float* Y, int32_t* acc_out,
                            float* gh_parts, int* nparts, int ppw, hipStream_t s) {
  constexpr int BM = 16 * TM, BN = 16 * TN;
  const int64_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  const size_t lds = (size_t)W * NB * TM * TN * 64 * 16 + 3 * 4 * BM;
  static bool once = ((void)hipFuncSetAttribute(
                          reinterpret_cast<const void*>(mfma_ksplit_kernel<NB, TM, TN, W, CPW, EPI>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds),
                      true);
  (void)once;
  if (nparts) *nparts = (int)nbn;
  hipLaunchKernelGGL((mfma_ksplit_kernel<NB, TM, TN, W, CPW, EPI>), dim3((unsigned)(nbm * nbn)),
                     dim3(64 * W), lds, s, Xq, xs, rs, M, Kp, W0, s0, W1, s1, N, Y, acc_out,
                     gh_parts, (int)nbn, ppw);
  return hipGetLastError();
}

constexpr int kKsWaves = 8;      // waves per block
constexpr int64_t kKsBlocks = 256;  // blocks that fill the 256 CUs once
static int ks_ppw(int64_t Kp) {
  return (int)(((Kp + kPiece - 1) / kPiece + kKsWaves - 1) / kKsWaves);
}

// Pieces per wave held in registers: the smallest instance that covers Kp
// (at most 4: up to 80 VGPRs of loads per piece for the 64 x 32 gate/up tile).
template <int NB, int TM, int TN, int EPI, int MAXC = 4>
static hipError_t ksplit_cpw(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                             int64_t Kp, const uint32_t* W0, const float* s0, const uint32_t* W1,
                             const float* s1, int64_t N, float* Y, int32_t* acc_out,
                             float* gh_parts, int* nparts, hipStream_t s) {
  const int ppw = ks_ppw(Kp);
#define BL_KS_GO(C)                                                                        \
  if ((C) <= MAXC && ppw <= (C))                                                           \
  return ksplit_go<NB, TM, TN, kKsWaves, ((C) <= MAXC ? (C) : 1), EPI>(                     \
      Xq, xs, rs, M, Kp, W0, s0, W1, s1, N, Y, acc_out, gh_parts, nparts, ppw, s)
  BL_KS_GO(1);
  BL_KS_GO(2);
  BL_KS_GO(3);
  BL_KS_GO(4);
#undef BL_KS_GO
  return hipErrorInvalidValue;
}

// Where this kernel measured faster than the kernels it replaces (same box,
// bit-identical results, events around graph replays):
// - 17..64 tokens, plain products: 6912 -> 2560 at 17 / 32 / 64 tokens 6.8 /
//   7.3 / 8.8 us against 9.4 / 9.7 / 9.9 for the 32 x 32 block-tile kernel,
//   2560 -> 6912 at 17 / 32 / 64 tokens 6.1 / 6.2 / 7.7 against 6.2 / 6.4 / 8.4;
// - 2..16 tokens, plain products with K <= 4096 and 4096..16384 columns:
//   2560 -> 6912 at 2 / 8 / 16 tokens 4.1 / 4.7 / 5.1 us against 4.7 / 5.5 /
//   6.3 for the direct and streaming kernels; at 2 tokens with longer K too
//   (6912 -> 2560: 4.5 against 5.0 us; at 4 and 8 tokens about even alone but
//   the FFN block, whose down projection this is, 0.2 / 0.5 us slower, and at
//   16 tokens 6.7 against 6.3 us, so from 3 tokens on the direct kernel);
// - the FFN's gate/up at 17..64 tokens: the block at 17 / 32 / 48 / 64
//   tokens 22.7 / 24.4 / 26.8 / 29.0 us against 27.6 / 28.7 / 30.2 / 30.7
//   with the block-tile kernel (both products).
// Measured slower and left to the other kernels: gate/up at 2..16 tokens (the
// FFN block 0.4-1.6 us slower), and the 100B-class layer (two to three times
// slower than the streaming kernel with pieces of 128).  Layers of more than
// 16384 or fewer than 2048 columns were not measured and stay where they were.
bool ksplit_ok(int64_t M, int64_t K, int64_t N, int nb) {
  const int64_t Kp = (K + 63) / 64 * 64;
  // the FFN's gate/up past 64 tokens: the block at 65 / 96 / 128 / 192 tokens
  // 35.8 / 39.4 / 47.5 / 57.8 us against 51.9 / 53.8 / 60.7 / 61.1 with the
  // 128 x 128 block-tile gate/up (at 256 / 512 tokens 74.5 / 115.5 against
  // 70.2 / 85.1, left to it)
  if (nb == 2 && M > 64) return M <= 192 && ks_ppw(Kp) <= 4 && N >= 2048 && N <= 16384;
  // 65..384 tokens, plain products: where the tiled GEMM has few tiles (same
  // box, events; 2560 -> 6912 at 65 / 128 / 192 / 256 tokens 10.7 / 11.3 /
  // 15.9 / 20.5 us against 23.0 / 20.9 / 22.5 / 20.6 on 128 x 256 tiles and
  // 18.1 at 256 on 128 x 128; 6912 -> 2560 at 65 / 128 / 256 / 384 / 512
  // tokens 8.9 / 15.6 / 22.0 / 29.0 / 36.0 against 44.4 / 42.3 / 41.8 / 41.8 /
  // 42.2 on 128 x 256 tiles and 33.7 on 128 x 128 at 768): up to 192 tokens,
  // and up to 384 with K of 4096 or more
  if (nb == 1 && M > 64)
    return (M <= 192 || (M <= 384 && Kp >= 4096)) && ks_ppw(Kp) <= 4 && N >= 2048 &&
           N <= 16384;
  if (M < 2 || M > 64 || ks_ppw(Kp) > 4 || N < 2048 || N > 16384) return false;
  if (nb == 2) return M >= 17;
  if (M == 2) return true;
  if (M <= 16) return Kp <= 4096 && N >= 4096;
  return true;
}

// Tiles: the narrowest of 16 x 16, 16 x 32, 16 x 48, 16 x 64 that gives at
// most one block per CU, else 32 x 64.  (With pieces of 128 weights, 16 x 32
// against 16 x 48 tiles for 6912 -> 2560 at 17 / 32 / 48 tokens: 7.6 / 8.4 /
// 8.4 against 9.2 / 10.2 / 10.2 us; at 64 tokens, 320 blocks of 16 x 32, 12.7
// against 10.3 us.)
hipError_t launch_ksplit(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                         int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                         int32_t* acc_out, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  const int64_t nbm = (M + 15) / 16;
#define BL_KS_TILE(TM_, TN_, MAXC_)                                                          \
  return ksplit_cpw<1, TM_, TN_, KS_STORE, MAXC_>(Xq, xs, rs, M, Kp, Wp, ws, nullptr, nullptr, \
                                                  N, Y, acc_out, nullptr, nullptr, s)
  if (M > 64) {
    // the tile (up to 64 x 64, within the register budget of its pieces per
    // wave) that moves the fewest bytes through the busiest CU
    struct Cand { int tm, tn, maxc; };
    static const Cand cands[] = {{1, 2, 4}, {1, 4, 4}, {2, 2, 4}, {2, 4, 2}, {4, 2, 2}, {4, 4, 2}};
    const int ppw = ks_ppw(Kp);
    int best = -1;
    int64_t bb = 0;
    for (int i = 0; i < 6; ++i) {
      if (ppw > cands[i].maxc) continue;
      const int64_t bm = 16 * cands[i].tm, bn = 16 * cands[i].tn;
      const int64_t blocks = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
      const int64_t bytes = (blocks + kKsBlocks - 1) / kKsBlocks * (bm * Kp + bn * (Kp / 4));
      if (best < 0 || bytes < bb) best = i, bb = bytes;
    }
    switch (best) {
      case 0: BL_KS_TILE(1, 2, 4);
      case 1: BL_KS_TILE(1, 4, 4);
      case 2: BL_KS_TILE(2, 2, 4);
      case 3: BL_KS_TILE(2, 4, 2);
      case 4: BL_KS_TILE(4, 2, 2);
      default: BL_KS_TILE(4, 4, 2);
    }
  }
  if (nbm * ((N + 15) / 16) <= kKsBlocks) BL_KS_TILE(1, 1, 4);
  if (nbm * ((N + 31) / 32) <= kKsBlocks) BL_KS_TILE(1, 2, 4);
  if (nbm * ((N + 47) / 48) <= kKsBlocks) BL_KS_TILE(1, 3, 4);
  if (nbm * ((N + 63) / 64) <= kKsBlocks) BL_KS_TILE(1, 4, 4);
  if (((M + 31) / 32) * ((N + 63) / 64) <= kKsBlocks && ks_ppw(Kp) <= 2) BL_KS_TILE(2, 4, 2);
  BL_KS_TILE(1, 3, 4);
#undef BL_KS_TILE
}

hipError_t launch_ksplit_gateup(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                                int64_t K, const uint32_t* Wg, const float* sg,
                                const uint32_t* Wu, const float* su, int64_t N, float* H,
                                float* gh_parts, int* nparts, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  // 32 x 32 tiles of both matrices up to 32 tokens, 64 x 32 above (the FFN
  // at 48 / 64 tokens 26.8 / 29.0 us against 28.1 / 30.2 with the block-tile
  // gate/up kernel)
  if (M > 32 && ks_ppw(Kp) <= 2)  // 64 x 32 tiles: more pieces per wave spill
    return ksplit_cpw<2, 4, 2, KS_GATEUP, 2>(Xq, xs, rs, M, Kp, Wg, sg, Wu, su, N, H, nullptr,
                                          gh_parts, nparts, s);
  return ksplit_cpw<2, 2, 2, KS_GATEUP>(Xq, xs, rs, M, Kp, Wg, sg, Wu, su, N, H, nullptr,
                                        gh_parts, nparts, s);
}

}  // namespace bl

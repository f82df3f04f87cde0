// Ternary x int8 matrix product on the gfx950 matrix cores (MFMA), for more
// than one token: Y[m][n] = dequant(sum_k q[m][k] * t[n][k]).
//
// youngju.dev "BitNet論文分析", section "BitNet b1.58": the integer product is
// F.linear(x_q, w_q) followed by output * (w_scale * x_scale) / Q.
// dashen-tech "BitNet.cpp 深度解析" §3.1: it equals sum_pos - sum_neg.  With
// many tokens it is a dense contraction, so it runs on
// v_mfma_i32_16x16x64_i8 in the shifted-code form
//   acc = sum_k q[m][k] * (t[n][k] + 1) - rowsum[m],
// where a 2-bit word unpacks into an MFMA operand with four shift+mask ops:
// word j of a row holds weight 16j + 4s + b in byte b at bits 2s, so
// (w >> 2s) & 0x03030303 are the codes of weights 16j+4s..16j+4s+3 in order.
//
// Tiling: a 256-thread block (4 waves, WAVES_M x WAVES_N) computes a
// BM x BN tile of Y, BM = 16*TM*WAVES_M, BN = 16*TN*WAVES_N; each wave owns
// TM x TN 16x16 accumulator tiles.  K advances in chunks of 256: the
// activation chunk (BM x 256 int8) is staged through LDS (double buffered,
// one barrier per chunk); the packed weight chunk (16 bytes per lane per
// 16-row tile) goes straight from memory to registers and is unpacked there.
// Both are prefetched one chunk ahead.
//
// MFMA operand mapping (lane l, g = l / 16): A lane l supplies token row
// l % 16 and B lane l weight row l % 16, each with 16 k-values; result lane
// l, register r holds (token 4g + r, weight row l % 16).  In k-step s of a
// chunk, lane group g uses packed word 4g + s of the chunk (weights
// 16(4g+s) .. +15) and the matching 16 activation bytes at offset 64g + 16s.
#include "bl_device.h"
#include "bl_launch.h"
#include "gemm_tiles.h"

namespace bl {

// MF_A48: a4.8 codes stacked as 2 Mh rows (the int4 rows of Mh tokens, then
// their int8 rows); the streaming kernel forms y of the Mh tokens itself.
enum { MF_STORE = 0, MF_GATEUP = 1, MF_A48 = 2 };

hipError_t launch_mfma32(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                         int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                         int32_t* acc_out, hipStream_t s);
hipError_t launch_tiled_gateup(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                               int64_t K, const uint32_t* Wg, const float* sg, const uint32_t* Wu,
                               const float* su, int64_t N, float* H, float* gh_parts, int* nparts,
                               hipStream_t s);

constexpr int kChunk = 256;         // K per chunk
constexpr int kLdsPitch = 256 + 16; // bytes per staged activation row

// KS > 1 splits K inside the block: KS groups of the 4 waves, group kg taking
// chunks kg, kg + KS, ... of the same tile (each group its own LDS stages),
// and the groups' partial accumulators are added through LDS before the
// epilogue -- KS times as many waves in flight for layers with few output
// tiles and long K (the FFN's down projection: 6912 -> 2560 at 64 tokens,
// 160 tiles of 32 x 32).  This replaced a split-K kernel whose int32
// partials went through the workspace to a second launch: the FFN at 17
// to 48 tokens measured 27.7-29.9 us this way against 27.6-32.7 us.
template <int TM, int TN, int WAVES_M, int WAVES_N, int EPI, int P, int KS = 1>
__global__ __launch_bounds__(256 * KS) void mfma_gemm_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int64_t M, int64_t Kp,
    const uint32_t* __restrict__ W0, const float* __restrict__ s0,
    const uint32_t* __restrict__ W1, const float* __restrict__ s1, int64_t N,
    float* __restrict__ Y, int32_t* __restrict__ acc_out, float* __restrict__ gh_parts,
    int nbn) {
  static_assert(WAVES_M * WAVES_N == 4, "4 waves per K group");
  constexpr int NT = 256 * KS;
  constexpr int BM = 16 * TM * WAVES_M;
  constexpr int BN = 16 * TN * WAVES_N;
  constexpr int NB = (EPI == MF_GATEUP) ? 2 : 1;       // weight matrices
  constexpr int A_U4 = BM * (kChunk / 16) / 256;       // uint4 per thread per chunk
  constexpr int A_U4_PAD = A_U4 > 0 ? A_U4 : 1;
  __shared__ __attribute__((aligned(16))) int8_t lds_a[2][KS][BM * kLdsPitch];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kg = wave >> 2, wl = wave & 3;           // K group, wave within it
  const int gtid = tid & 255;                        // thread within the K group
  const int wm = wl / WAVES_N, wn = wl % WAVES_N;
  const int g = lane >> 4, li = lane & 15;
  const int bn = blockIdx.x % nbn, bm = blockIdx.x / nbn;
  const int64_t m0 = (int64_t)bm * BM, n0 = (int64_t)bn * BN;
  const int64_t wpr = Kp / 16;
  const int64_t nchunks = (Kp + kChunk - 1) / kChunk;
  const int64_t nsteps = (nchunks + KS - 1) / KS;    // chunks per K group (upper bound)

  TokenOperands<TM> tok;  // the epilogue's scales and row sums
  tok.load(x_scale, rowsum, M, m0 + 16 * wm * TM);
  const float ws0 = s0[0], ws1 = NB == 2 ? s1[0] : 0.0f;  // weight scales, also early

  // ---- loaders: P chunks of loads in flight, in registers.  Buffer loads
  // issued without branches: rows past M, words past a row's end and chunks
  // past K read as zero (zero codes, zero activations), so the compiler
  // waits for one chunk's loads at a time.
  static_assert(P >= 1, "at least one chunk in flight");
  const int64_t mrows = M - m0 < BM ? M - m0 : BM;  // rows of this block
  const int64_t nrows = N - n0 < BN ? N - n0 : BN;
  const buf_rsrc ra = make_buf_rsrc(Xq + m0 * Kp, (uint32_t)(mrows * Kp));
  const buf_rsrc rb0 = make_buf_rsrc(W0 + n0 * wpr, (uint32_t)(nrows * wpr * 4));
  const buf_rsrc rb1 = make_buf_rsrc((NB == 2 ? W1 : W0) + n0 * wpr, (uint32_t)(nrows * wpr * 4));
  u32x4 a_reg[P][A_U4_PAD];
  u32x4 b_reg[P][NB][TN];
  // step t of group kg is chunk t * KS + kg
  auto load = [&](int64_t t, int slot) {
    const int64_t kc = (t * KS + kg) * kChunk;
#pragma unroll
    for (int i = 0; i < A_U4_PAD; ++i) {
      const int u = gtid + 256 * i;
      const int row = u >> 4, c16 = u & 15;
      const int64_t k = kc + 16 * c16;
      const bool ok = row < BM && row < mrows && k < Kp;
      a_reg[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(
          ra, ok ? (uint32_t)(row * Kp + k) : 0x80000000u, 0, 0);
    }
    const int64_t word = kc / 16 + 4 * g;
#pragma unroll
    for (int mat = 0; mat < NB; ++mat) {
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) {
        // rows past N are past the resource's range and read as zero; the
        // weights are cached (the WAVES_M waves and the row blocks of the
        // grid read them again)
        const int64_t nl = 16 * (wn * TN + tn) + li;
        b_reg[slot][mat][tn] = __builtin_amdgcn_raw_buffer_load_b128(
            mat == 0 ? rb0 : rb1, word < wpr ? (uint32_t)((nl * wpr + word) * 4) : 0x80000000u, 0, 0);
      }
    }
  };
  auto store_a = [&](int buf, int slot) {
#pragma unroll
    for (int i = 0; i < A_U4_PAD; ++i) {
      const int u = gtid + 256 * i;
      const int row = u >> 4, c16 = u & 15;
      if (A_U4 > 0 || row < BM)
        *reinterpret_cast<u32x4*>(&lds_a[buf][kg][row * kLdsPitch + 16 * c16]) = a_reg[slot][i];
    }
  };

  v4i acc[NB][TM][TN];
#pragma unroll
  for (int mat = 0; mat < NB; ++mat)
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn) acc[mat][tm][tn] = v4i{0, 0, 0, 0};

#pragma unroll
  for (int d = 0; d < P; ++d) {
    load(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int64_t tb = 0; tb < nsteps; tb += P) {
#pragma unroll
    for (int d = 0; d < P; ++d) {
      const int64_t t = tb + d;
      const bool live = t < nsteps;  // uniform over the block
      const int buf = (int)(t & 1);
      if (live) store_a(buf, d);
      u32x4 b_cur[NB][TN];
#pragma unroll
      for (int mat = 0; mat < NB; ++mat)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) b_cur[mat][tn] = b_reg[d][mat][tn];
      if (live) __syncthreads();
      // refill the slot with step t + P (zeros past the end), then compute
      // (a group's step past the last chunk computes on zeros)
      load(t + P, d);
      __builtin_amdgcn_sched_barrier(0);
      if (live) {
        const int8_t* la = &lds_a[buf][kg][0];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v4i a[TM];
#pragma unroll
          for (int tm = 0; tm < TM; ++tm) {
            const int row = 16 * (wm * TM + tm) + li;
            a[tm] = *reinterpret_cast<const v4i*>(la + row * kLdsPitch + 64 * g + 16 * s);
          }
#pragma unroll
          for (int mat = 0; mat < NB; ++mat) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
              const v4i b = codes_operand(b_cur[mat][tn][s]);
#pragma unroll
              for (int tm = 0; tm < TM; ++tm)
                acc[mat][tm][tn] =
                    __builtin_amdgcn_mfma_i32_16x16x64_i8(a[tm], b, acc[mat][tm][tn], 0, 0, 0);
            }
          }
        }
      }
    }
  }

  // K groups 1 .. KS-1 hand their partial tiles to group 0 through the
  // (now free) activation stages
  if constexpr (KS > 1) {
    static_assert((KS - 1) * 4 * NB * TM * TN * 64 * 16 <= 2 * KS * BM * kLdsPitch,
                  "partial tiles fit in the activation stages");
    v4i* part = reinterpret_cast<v4i*>(&lds_a[0][0][0]);
    __syncthreads();  // every group is done reading the stages
    if (kg > 0) {
#pragma unroll
      for (int mat = 0; mat < NB; ++mat)
#pragma unroll
        for (int tm = 0; tm < TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < TN; ++tn)
            part[((((kg - 1) * 4 + wl) * NB + mat) * TM + tm) * TN * 64 + tn * 64 + lane] =
                acc[mat][tm][tn];
    }
    __syncthreads();
    if (kg == 0) {
#pragma unroll
      for (int k = 1; k < KS; ++k)
#pragma unroll
        for (int mat = 0; mat < NB; ++mat)
#pragma unroll
          for (int tm = 0; tm < TM; ++tm)
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
              acc[mat][tm][tn] +=
                  part[((((k - 1) * 4 + wl) * NB + mat) * TM + tm) * TN * 64 + tn * 64 + lane];
    }
  }
  const bool owner = kg == 0;

  // ---- epilogue (group 0)
  if constexpr (EPI == MF_STORE) {
    if (!owner) return;
    const float sw = ws0;
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = m0 + 16 * (wm * TM + tm) + 4 * g + r;
        if (m >= M) continue;
        const int32_t rsm = tok.rs[tm][r];
        const float sc = __fmul_rn(sw, tok.xs[tm][r]);
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
          const int64_t n = n0 + 16 * (wn * TN + tn) + li;
          if (n < N) {
            const int a = acc[0][tm][tn][r] - rsm;
            if (Y) Y[m * N + n] = dequant_fast(a, sc);
            if (acc_out) acc_out[m * N + n] = a;
          }
        }
      }
    }
  } else {
    __shared__ float red[WAVES_N][BM];
    const float sg = ws0, su = ws1;
    if (owner) {
#pragma unroll
      for (int tm = 0; tm < TM; ++tm) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int lrow = 16 * (wm * TM + tm) + 4 * g + r;
          const int64_t m = m0 + lrow;
          float hmax = 0.0f;
          if (m < M) {
            const int32_t rsm = tok.rs[tm][r];
            const float xs = tok.xs[tm][r];
            const float scg = __fmul_rn(sg, xs), scu = __fmul_rn(su, xs);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
              const int64_t n = n0 + 16 * (wn * TN + tn) + li;
              if (n < N) {
                const float gv = dequant_fast(acc[0][tm][tn][r] - rsm, scg);
                const float uv = dequant_fast(acc[1][tm][tn][r] - rsm, scu);
                const float a = gv > 0.0f ? gv : 0.0f;
                const float h = __fmul_rn(__fmul_rn(a, a), uv);
                Y[m * N + n] = h;
                hmax = fmaxf(hmax, fabsf(h));
              }
            }
          }
          // max over the 16 lanes holding this row
#pragma unroll
          for (int o = 8; o > 0; o >>= 1) hmax = fmaxf(hmax, __shfl_xor(hmax, o));
          if (li == 0) red[wn][lrow] = hmax;
        }
      }
    }
    __syncthreads();
    for (int lrow = tid; lrow < BM; lrow += NT) {
      float v = red[0][lrow];
#pragma unroll
      for (int w = 1; w < WAVES_N; ++w) v = fmaxf(v, red[w][lrow]);
      const int64_t m = m0 + lrow;
      if (m < M) gh_parts[(int64_t)bn * M + m] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Few tokens (M <= 16), weights streamed from HBM.
//
// The activation block (M x Kp int8) is copied into LDS once.  Each wave owns
// 16 weight rows (one 16x16 MFMA tile; token rows M..15 are fed as zeros).
// The weights are read the way the GEMV reads them -- every load instruction
// covers LPR lanes x 16 bytes of one row, contiguous -- because the MFMA
// operand layout (16 rows x 64 bytes per instruction) measured ~50 % slower
// from HBM.  Each step of STEP weights per row goes registers -> a
// wave-private LDS patch -> MFMA operands: lane (g, li) takes row li, words
// 4g .. 4g+3 of each 256-weight block (k-step s uses word 4g + s and the
// activation bytes at 64g + 16s of the block).  D steps of loads are in
// flight while a step is computed.  NB = 2 runs the FFN's gate and up
// weights together.
//
// KS > 1 splits K: the KS waves of a tile take consecutive ranges of steps
// and the partial accumulators of waves 1 .. KS-1 are added to wave 0's
// through LDS before the epilogue (more waves in flight for layers with few
// rows, e.g. the FFN's down projection).
template <int NB, int LPR, int WPB, int D, int EPI, int KS, int BITS = 2, bool PH = false>
__global__ __launch_bounds__(64 * WPB) void mfma_stream_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ x_scale,
    const int32_t* __restrict__ rowsum, int M, int64_t Kp, int64_t Kw,
    const uint32_t* __restrict__ W0, const float* __restrict__ s0,
    const uint32_t* __restrict__ W1, const float* __restrict__ s1, int64_t N,
    float* __restrict__ Y, int32_t* __restrict__ acc_out, float* __restrict__ gh_parts,
    int sph) {
  static_assert(BITS == 2 || BITS == 1, "2-bit codes or the 1-bit binary layout");
  constexpr int STEP = LPR * 64 * (2 / BITS);    // weights per row per step (16 B per lane)
  constexpr int RPI = 64 / LPR;                  // rows per load instruction
  constexpr int NI = 16 / RPI;                   // load instructions per matrix per step
  constexpr int BP = STEP * BITS / 8 + 16;       // bytes per staged weight row (+ pad)
  constexpr int TPB = WPB / KS;                  // 16-row tiles per block
  static_assert(TPB * KS == WPB, "KS divides WPB");
  extern __shared__ __attribute__((aligned(16))) int8_t lds[];
  __shared__ float red[WPB][16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = wave / KS, kpart = wave % KS;
  const int g = lane >> 4, li = lane & 15;
  // PH: the activations are staged sph steps at a time (M x Kp does not fit
  // next to the weight patches); otherwise all of K at once
  const int64_t kph = PH && (int64_t)sph * STEP < Kp ? (int64_t)sph * STEP : Kp;
  const int64_t pitch = kph + 16;                // staged activation row
  int8_t* lds_x = lds;
  const int64_t xbytes = staged_rows_bytes(M, pitch);
  int8_t* lds_w = lds + xbytes + (int64_t)wave * NB * 16 * BP;
  v4i* lds_part = reinterpret_cast<v4i*>(lds + xbytes + (int64_t)WPB * NB * 16 * BP);
  // weight rows hold Kw weights (Kp for 2-bit codes, Kp rounded up to 128 for
  // the 1-bit layout)
  const int64_t wpr = Kw * BITS / 32;
  const int C = (int)(Kw * BITS / 128);          // 16-byte pieces per row
  const int nsteps_all = (int)((Kw + STEP - 1) / STEP);
  const int s_begin = kpart * nsteps_all / KS, s_end = (kpart + 1) * nsteps_all / KS;
  const int nsteps = s_end - s_begin;            // this wave's steps
  const int64_t nbase = (int64_t)blockIdx.x * (16 * TPB) + 16 * tile;  // first row of the tile
  const int lr = lane / LPR, lc = lane % LPR;    // load role: row-in-instruction, piece

  // D steps of weights in flight, in registers.  Every load is issued
  // unconditionally (a buffer load): pieces past the row's end (k >= Kw) and
  // steps past this wave's range get an offset outside the buffer and read as
  // zero without touching memory.  Zero codes there meet zero activation
  // bytes (the operand reads below are zeroed for k >= Kp), and with no
  // branches the compiler waits for one step's loads at a time.
  uint4 st[D][NB][NI];
  const buf_rsrc wr0 = make_buf_rsrc(W0, (uint32_t)(N * wpr * 4));
  const buf_rsrc wr1 = make_buf_rsrc(NB == 2 ? W1 : W0, (uint32_t)(N * wpr * 4));
  uint32_t row_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    int64_t n = nbase + RPI * i + lr;
    n = n < N ? n : N - 1;
    row_off[i] = (uint32_t)(n * wpr * 4);
  }
  auto load_step = [&](int sidx, uint4 (&dst)[NB][NI]) {
    const int c = (s_begin + sidx) * LPR + lc;
    const bool ok = sidx < nsteps && c < C;
#pragma unroll
    for (int mat = 0; mat < NB; ++mat) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const uint32_t off = ok ? row_off[i] + 16u * (uint32_t)c : 0x80000000u;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(mat == 0 ? wr0 : wr1, off, 0, 2);
        dst[mat][i] = make_uint4(v[0], v[1], v[2], v[3]);
      }
    }
  };
  auto stage_step = [&](const uint4 (&src)[NB][NI]) {
#pragma unroll
    for (int mat = 0; mat < NB; ++mat)
#pragma unroll
      for (int i = 0; i < NI; ++i)
        *reinterpret_cast<uint4*>(lds_w + (mat * 16 + RPI * i + lr) * BP + 16 * lc) = src[mat][i];
  };
  auto wave_sync = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // the epilogue's per-token scales and row sums first (the oldest loads:
  // the wait for the activations below covers them); MF_A48 also the int8
  // rows' scales
  TokenOperands<1> tok;
  tok.load(x_scale, rowsum, M, 0);
  const float ws0 = s0[0], ws1 = EPI == MF_GATEUP ? s1[0] : 0.0f;  // weight scales
  float xs8[4] = {};
  if constexpr (EPI == MF_A48) {
    const buf_rsrc rx = make_buf_rsrc(x_scale, (uint32_t)(4 * M));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      xs8[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          rx, m < M / 2 ? (uint32_t)(4 * (m + M / 2)) : 0x80000000u, 0, 0));
    }
  }

  // activations -> LDS, every load in flight at once; then the first D steps
  // of weights, so that waiting for the activations (the older loads) leaves
  // the weight steps in flight and the loop starts in the state it repeats
  stage_rows_lds<64 * WPB>(Xq, Kp, M, 0, (int)kph, (int)pitch, lds_x);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int d = 0; d < D; ++d) load_step(d, st[d]);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(D * NB * NI));
  __syncthreads();

  v4i acc[NB][2];
#pragma unroll
  for (int mat = 0; mat < NB; ++mat) acc[mat][0] = acc[mat][1] = v4i{0, 0, 0, 0};
  const bool arow = li < M;
  const int8_t* xrow = lds_x + (arow ? li : 0) * pitch + 64 * g;
  int64_t xbase = 0;   // K position of the first staged column
  int next_ph = sph;   // step at which the next phase is staged

  for (int sbase = 0; sbase < nsteps; sbase += D) {
#pragma unroll
  for (int d = 0; d < D; ++d) {
    // no early exit from this unrolled loop: a step past the end (the last
    // trip's tail) stages and loads like any other (out-of-range reads are
    // zero) and skips its dot products, so the loop has one latch and the
    // compiler keeps the later steps' loads in flight across it
    const int sidx = sbase + d;
    const bool live = sidx < nsteps;  // uniform over the wave (and block)
    const int sabs = s_begin + sidx;
    if (PH && live && sabs == next_ph) {
      // next phase of the activations (KS == 1 only: every wave of the block
      // is at the same step); the weight patches are wave-private
      __syncthreads();
      xbase = (int64_t)sabs * STEP;
      stage_rows_lds<64 * WPB>(Xq, Kp, M, xbase, (int)(Kp - xbase < kph ? Kp - xbase : kph),
                               (int)pitch, lds_x);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      next_ph += sph;
    }
    stage_step(st[d]);
    wave_sync();
    load_step(sidx + D, st[d]);
    __builtin_amdgcn_sched_barrier(0);
    const int64_t k0 = (int64_t)sabs * STEP;
    const int64_t kx = PH ? k0 - xbase : k0;  // k0 within the staged phase
#pragma unroll
    for (int b = 0; b < STEP / 256; ++b) {
      if (live && k0 + 256 * b < Kw) {
        // this lane's 64 weights of the 256-weight block: 16 bytes of codes
        // or 8 bytes of bits
        uint4 bw[NB];
#pragma unroll
        for (int mat = 0; mat < NB; ++mat) {
          const int8_t* pw = lds_w + (mat * 16 + li) * BP;
          if constexpr (BITS == 2) {
            bw[mat] = *reinterpret_cast<const uint4*>(pw + 64 * b + 16 * g);
          } else {
            const uint2 h = *reinterpret_cast<const uint2*>(pw + 32 * b + 8 * g);
            bw[mat] = make_uint4(h.x, h.y, 0u, 0u);
          }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          // this lane's activation bytes, read unconditionally: token rows
          // li >= M read row 0 and only feed result rows that are dropped,
          // and bytes past Kp (the next staged row, or the weight patches
          // after the last row) meet weight codes that are zero there --
          // pieces past the row end load as zero
          const v4i a = *reinterpret_cast<const v4i*>(xrow + kx + 256 * b + 16 * s);
#pragma unroll
          for (int mat = 0; mat < NB; ++mat) {
            v4i bv;
            if constexpr (BITS == 2) {
              bv = codes_operand(s == 0 ? bw[mat].x : s == 1 ? bw[mat].y : s == 2 ? bw[mat].z : bw[mat].w);
            } else {
              const uint32_t wd = s < 2 ? bw[mat].x : bw[mat].y;
              bv = (s & 1) ? bits_operand<1>(wd) : bits_operand<0>(wd);
            }
            acc[mat][s & 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, bv, acc[mat][s & 1], 0, 0, 0);
          }
        }
      }
    }
    wave_sync();
  }
  }

  // K split: fold the partial sums of waves 1 .. KS-1 into wave 0 of the tile
#pragma unroll
  for (int mat = 0; mat < NB; ++mat) acc[mat][0] += acc[mat][1];
  if constexpr (KS > 1) {
    if (kpart > 0) {
#pragma unroll
      for (int mat = 0; mat < NB; ++mat)
        lds_part[((tile * (KS - 1) + kpart - 1) * NB + mat) * 64 + lane] = acc[mat][0];
    }
    __syncthreads();
    if (kpart == 0) {
#pragma unroll
      for (int k = 1; k < KS; ++k)
#pragma unroll
        for (int mat = 0; mat < NB; ++mat)
          acc[mat][0] += lds_part[((tile * (KS - 1) + k - 1) * NB + mat) * 64 + lane];
    }
  }
  const bool owner = kpart == 0;

  // result lane l, register r: token 4g + r, weight row nbase + li
  const int64_t n = nbase + li;
  if constexpr (EPI == MF_STORE) {
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
  } else if constexpr (EPI == MF_A48) {
    // rows m and m + Mh of the tile are token m's int4 and int8 parts; the
    // wave trades its accumulators through its own weight patch (free after
    // the last step) so the lane of row m sees both
    const float sw = ws0;
    const int Mh = M / 2;
    int av[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      av[r] = m < M ? acc[0][0][r] - tok.rs[0][r] : 0;
      if (owner && m < M && n < N && acc_out) acc_out[(int64_t)m * N + n] = av[r];
    }
    int* ex = reinterpret_cast<int*>(lds_w);
    wave_sync();
#pragma unroll
    for (int r = 0; r < 4; ++r) ex[(4 * g + r) * 16 + li] = av[r];
    wave_sync();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (owner && m < Mh && n < N)
        Y[(int64_t)m * N + n] = a48_dequant(av[r], __fmul_rn(sw, tok.xs[0][r]),
                                            ex[(m + Mh) * 16 + li], __fmul_rn(sw, xs8[r]));
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
        const float uv = dequant_fast(acc[1][0][r] - rsm, __fmul_rn(su, xs));
        const float t = gv > 0.0f ? gv : 0.0f;
        const float h = __fmul_rn(__fmul_rn(t, t), uv);
        Y[(int64_t)m * N + n] = h;
        hm = fabsf(h);
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) hm = fmaxf(hm, __shfl_xor(hm, o));
      if (li == 0) red[wave][m] = hm;
    }
    __syncthreads();
    if (tid < 16 && tid < M) {
      float v = red[0][tid];
#pragma unroll
      for (int w = 1; w < WPB; ++w) v = fmaxf(v, red[w][tid]);
      gh_parts[(int64_t)blockIdx.x * M + tid] = v;
    }
  }
}

// Activation bytes the streaming kernel may stage in LDS.
constexpr int64_t kStreamLds = 144 * 1024;
constexpr int64_t kCUs = 256;  // compute units of the MI355X

// the activation block plus one wave's weight patches (two matrices)
static bool stream_ok(int64_t M, int64_t Kp) {
  return M <= 16 && M * (Kp + 16) + 2 * 16 * (32 * 16 + 16) <= kStreamLds;
}

// Dynamic LDS above 64 KiB has to be allowed per kernel once.
template <typename Kern>
static void allow_lds(Kern k) {
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kStreamLds);
}

// 16 lanes (256 contiguous bytes) per weight row and load: measured against
// 32 lanes 17.6 -> 15.9 us on the 100B-class layer at 8 tokens (8 lanes
// about the same, 4 lanes slower); deeper load pipelines (D > 1) were slower
constexpr int kStreamLpr = 16;
constexpr int kStreamBp = kStreamLpr * 16 + 16;  // staged bytes per weight row and step

// kx: activation columns staged at a time (Kp, or a phase of whole steps)
static int64_t stream_lds_bytes(int64_t M, int64_t kx, int nb, int wpb, int ks) {
  return staged_rows_bytes(M, kx + 16) + (int64_t)wpb * nb * 16 * kStreamBp +
         (int64_t)(wpb / ks) * (ks - 1) * nb * 1024;
}

// Large layers (>= 1600 tiles of 16 rows) at up to 16 tokens whose M x Kp
// activations do not fit next to 8 waves' weight patches: staged in phases.
static bool stream_phased_ok(int64_t M, int64_t N) { return M <= 16 && (N + 15) / 16 >= 200 * 8; }

template <int NB, int WPB, int KS, int EPI, int BITS, bool PH = false>
static hipError_t stream_go(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                            int64_t Kp, int64_t Kw, const uint32_t* W0, const float* s0,
                            const uint32_t* W1, const float* s1, int64_t N, float* Y,
                            int32_t* acc_out, float* gh_parts, int* nparts, hipStream_t s,
                            int sph, int64_t kx) {
  constexpr int TPB = WPB / KS;
  const size_t lds = (size_t)stream_lds_bytes(M, kx, NB, WPB, KS);
  const unsigned blocks = (unsigned)((N + 16 * TPB - 1) / (16 * TPB));
  if (nparts) *nparts = (int)blocks;
  // steps of weights in flight per wave: 2 and 3 measured no faster (3 slower)
  // on the 100B-class layer at 8 and 16 tokens -- the kernel is bound by its
  // per-wave unpack, LDS operand reads and MFMA chains, not by load latency
  constexpr int D = 1;
  static bool once =
      (allow_lds(mfma_stream_kernel<NB, kStreamLpr, WPB, D, EPI, KS, BITS, PH>), true);
  (void)once;
  hipLaunchKernelGGL((mfma_stream_kernel<NB, kStreamLpr, WPB, D, EPI, KS, BITS, PH>), dim3(blocks),
                     dim3(64 * WPB), lds, s, Xq, xs, rs, (int)M, Kp, Kw, W0, s0, W1, s1, N, Y,
                     acc_out, gh_parts, sph);
  return hipGetLastError();
}

// Tiles (16 weight rows) per block as keep about 200 blocks, most of the 256
// CUs busy (more tiles per block share one staged copy of the activations);
// layers with too few rows for that split K over 2 or 4 waves per tile.
// Large layers take 7 tiles per block instead of 8 when that still gives at
// most one block per CU and fills more CUs (the 100B-class layer: 256 blocks
// instead of 224, 15.2 us against 15.5 us at 8 tokens).
template <int NB, int EPI, int BITS = 2>
static hipError_t stream_launch(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                                int64_t Kp, const uint32_t* W0, const float* s0,
                                const uint32_t* W1, const float* s1, int64_t N, float* Y,
                                int32_t* acc_out, float* gh_parts, int* nparts, hipStream_t s) {
  const int64_t Kw = BITS == 2 ? Kp : (Kp + 127) / 128 * 128;  // weights per row
  auto fits = [&](int wpb, int ks) { return stream_lds_bytes(M, Kp, NB, wpb, ks) <= kStreamLds; };
  const int64_t tiles = (N + 15) / 16;
  constexpr int64_t STEP = 64 * kStreamLpr * (2 / BITS);
  const int64_t nsteps = (Kw + STEP - 1) / STEP;
  int sph = (int)nsteps;
  int64_t kx = Kp;
#define BL_STREAM_GO(WPB, KS)                                                                 \
  return stream_go<NB, WPB, KS, EPI, BITS>(Xq, xs, rs, M, Kp, Kw, W0, s0, W1, s1, N, Y,       \
                                           acc_out, gh_parts, nparts, s, sph, kx)
  const bool seven = (tiles + 6) / 7 <= kCUs && (tiles + 6) / 7 > (tiles + 7) / 8;
  if (tiles >= 200 * 8 && seven && fits(7, 1)) BL_STREAM_GO(7, 1);
  if (tiles >= 200 * 8 && fits(8, 1)) BL_STREAM_GO(8, 1);
  if (stream_phased_ok(M, N)) {
    // fewest phases that fit next to the waves' patches
    const int wpb = seven ? 7 : 8;
    for (int64_t P = 2; P <= nsteps; ++P) {
      sph = (int)((nsteps + P - 1) / P);
      kx = sph * STEP < Kp ? sph * STEP : Kp;
      if (stream_lds_bytes(M, kx, NB, wpb, 1) > kStreamLds) continue;
      if (wpb == 7)
        return stream_go<NB, 7, 1, EPI, BITS, true>(Xq, xs, rs, M, Kp, Kw, W0, s0, W1, s1, N, Y,
                                                    acc_out, gh_parts, nparts, s, sph, kx);
      return stream_go<NB, 8, 1, EPI, BITS, true>(Xq, xs, rs, M, Kp, Kw, W0, s0, W1, s1, N, Y,
                                                  acc_out, gh_parts, nparts, s, sph, kx);
    }
    sph = (int)nsteps;
    kx = Kp;
  }
  if (tiles >= 200 * 4 && fits(4, 1)) BL_STREAM_GO(4, 1);
  if (tiles >= 200 * 2 && fits(2, 1)) BL_STREAM_GO(2, 1);
  if (tiles >= 200 || nsteps < 2) BL_STREAM_GO(1, 1);
  if (nsteps >= 4 && fits(4, 4)) BL_STREAM_GO(4, 4);
  if (fits(2, 2)) BL_STREAM_GO(2, 2);
  BL_STREAM_GO(1, 1);
#undef BL_STREAM_GO
}

template <int TM, int TN, int WAVES_M, int WAVES_N, int EPI, int P = 1, int KS = 1>
static hipError_t mfma_launch(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                              int64_t Kp, const uint32_t* W0, const float* s0, const uint32_t* W1,
                              const float* s1, int64_t N, float* Y, int32_t* acc_out,
                              float* gh_parts, int* nparts, hipStream_t s) {
  constexpr int BM = 16 * TM * WAVES_M;
  constexpr int BN = 16 * TN * WAVES_N;
  const int64_t nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
  if (nparts) *nparts = (int)nbn;
  hipLaunchKernelGGL((mfma_gemm_kernel<TM, TN, WAVES_M, WAVES_N, EPI, P, KS>),
                     dim3((unsigned)(nbm * nbn)), dim3(256 * KS), 0, s, Xq, xs, rs, M, Kp, W0, s0, W1,
                     s1, N, Y, acc_out, gh_parts, (int)nbn);
  return hipGetLastError();
}

hipError_t launch_mfma(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M, int64_t K,
                       const uint32_t* Wp, const float* ws, int64_t N, float* Y, int32_t* acc_out,
                       bool tiled, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  if (tiled) return launch_mfma32(Xq, xs, rs, M, K, Wp, ws, N, Y, acc_out, s);
  // K split over the waves of a block, where that measured faster (ksplit_ok)
  if (ksplit_ok(M, K, N, 1)) return launch_ksplit(Xq, xs, rs, M, K, Wp, ws, N, Y, acc_out, s);
  if (M > 64) return launch_mfma32(Xq, xs, rs, M, K, Wp, ws, N, Y, acc_out, s);
  // large layers: the streaming kernel with 7- or 8-wave blocks (activations
  // staged in phases when they do not fit), 18.5 us against the direct
  // kernel's 39.5 us on the 100B-class layer at 16 tokens
  if (!stream_phased_ok(M, N) && direct_ok(M, K, N, 1))
    return launch_direct(Xq, xs, rs, M, K, Wp, ws, N, Y, acc_out, s);
  if (stream_ok(M, Kp) || stream_phased_ok(M, N))
    return stream_launch<1, MF_STORE>(Xq, xs, rs, M, Kp, Wp, ws, nullptr, nullptr, N, Y, acc_out,
                                      nullptr, nullptr, s);
  if (M <= 16)
    return mfma_launch<1, 1, 1, 4, MF_STORE>(Xq, xs, rs, M, Kp, Wp, ws, nullptr, nullptr, N, Y,
                                             acc_out, nullptr, nullptr, s);
  // 17 <= M <= 64: 32 x 32 block tiles (four 16 x 16 wave tiles) keep more
  // blocks in flight than 64-row tiles for these weight-streaming shapes,
  // with 2 chunks of loads in flight per wave; long K split over 4 groups of
  // waves in the block (6912 -> 2560 at 64 tokens: 9.9 us against 12.6 with
  // one group and 4 chunks in flight, 19.5 with one chunk; at 32 tokens the
  // same), shorter K over 2 groups up to 32 tokens (2560 -> 6912: 6.3 against
  // 6.7 us) and one group above (8.3 against 8.4 us at 64 tokens)
  if ((Kp + kChunk - 1) / kChunk >= 16)
    return mfma_launch<1, 1, 2, 2, MF_STORE, 2, 4>(Xq, xs, rs, M, Kp, Wp, ws, nullptr, nullptr, N,
                                                   Y, acc_out, nullptr, nullptr, s);
  if (M <= 32)
    return mfma_launch<1, 1, 2, 2, MF_STORE, 2, 2>(Xq, xs, rs, M, Kp, Wp, ws, nullptr, nullptr, N,
                                                   Y, acc_out, nullptr, nullptr, s);
  return mfma_launch<1, 1, 2, 2, MF_STORE, 2>(Xq, xs, rs, M, Kp, Wp, ws, nullptr, nullptr, N, Y,
                                              acc_out, nullptr, nullptr, s);
}

// The stacked a4.8 product (M2 = 2 Mh code rows) where launch_mfma runs the
// streaming kernel: that kernel then writes y too (no combine launch).
bool stream_a48_ok(int64_t M2, int64_t K, int64_t N) {
  const int64_t Kp = (K + 63) / 64 * 64;
  if (M2 > 16 || M2 % 2 != 0) return false;
  if (!stream_phased_ok(M2, N) && direct_ok(M2, K, N, 1)) return false;
  return stream_ok(M2, Kp) || stream_phased_ok(M2, N);
}

hipError_t launch_stream_a48(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M2,
                             int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                             int32_t* acc, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  return stream_launch<1, MF_A48>(Xq, xs, rs, M2, Kp, Wp, ws, nullptr, nullptr, N, Y, acc,
                                  nullptr, nullptr, s);
}

bool stream_1bit_ok(int64_t M, int64_t K, int64_t N) {
  return stream_ok(M, (K + 63) / 64 * 64) || stream_phased_ok(M, N);
}

hipError_t launch_stream_1bit(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                              int64_t K, const uint32_t* Wb, const float* ws, int64_t N, float* Y,
                              int32_t* acc_out, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  return stream_launch<1, MF_STORE, 1>(Xq, xs, rs, M, Kp, Wb, ws, nullptr, nullptr, N, Y, acc_out,
                                       nullptr, nullptr, s);
}

int64_t mfma_gateup_parts(int64_t M, int64_t N) {
  // the narrowest block used by launch_mfma_gateup covers 16 columns
  (void)M;
  return (N + 15) / 16;
}

hipError_t launch_mfma_gateup(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                              int64_t K, const uint32_t* Wg, const float* sg, const uint32_t* Wu,
                              const float* su, int64_t N, float* H, float* gh_parts, int* nparts,
                              hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  // the streaming kernel first: the 2B-class FFN block 20.4-20.8 -> 20.2-20.4
  // us at 8 tokens, 18.4-18.8 -> 18.2-18.3 at 2, 22.0-22.6 -> 22.0-22.4 at 16
  // against the direct kernel (two boxes)
  if (stream_ok(M, Kp))
    return stream_launch<2, MF_GATEUP>(Xq, xs, rs, M, Kp, Wg, sg, Wu, su, N, H, nullptr, gh_parts,
                                       nparts, s);
  if (direct_ok(M, K, N, 2))
    return launch_direct_gateup(Xq, xs, rs, M, K, Wg, sg, Wu, su, N, H, gh_parts, nparts, s);
  if (M <= 16)
    return mfma_launch<1, 1, 1, 4, MF_GATEUP>(Xq, xs, rs, M, Kp, Wg, sg, Wu, su, N, H, nullptr,
                                              gh_parts, nparts, s);
  // 17 <= M <= 64: 32 x 32 block tiles with 2 chunks of loads in flight
  // (the FFN at 64 tokens 35.2 us against 38.2 with 64 x 16 tiles and one
  // chunk in flight, at 32 tokens 28.7 against 33.7)
  // 17..192 tokens: K split over the waves of a block (ksplit_ok)
  if (ksplit_ok(M, K, N, 2))
    return launch_ksplit_gateup(Xq, xs, rs, M, K, Wg, sg, Wu, su, N, H, gh_parts, nparts, s);
  if (M <= 64)
    return mfma_launch<1, 1, 2, 2, MF_GATEUP, 2>(Xq, xs, rs, M, Kp, Wg, sg, Wu, su, N, H, nullptr,
                                                 gh_parts, nparts, s);
  // the tiled GEMM with both matrices once its 128 x 128 tiles fill the CUs
  // more than once (the FFN block at 1024 / 2048 tokens 121.6 / 207.2 ->
  // 105.3 / 168.9 us; at 193 / 256 / 512 tokens 1-2 us slower, so not there)
  if (((M + 127) / 128) * ((N + 127) / 128) > 256)
    return launch_tiled_gateup(Xq, xs, rs, M, K, Wg, sg, Wu, su, N, H, gh_parts, nparts, s);
  return mfma_launch<4, 4, 2, 2, MF_GATEUP>(Xq, xs, rs, M, Kp, Wg, sg, Wu, su, N, H, nullptr,
                                            gh_parts, nparts, s);
}

}  // namespace bl

namespace bl {

template <int TM, int TN, int WM, int WN>
static hipError_t tiled_go(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                           int64_t Kp, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                           int32_t* acc_out, hipStream_t s) {
  using G = TiledGemm<TM, TN, WM, WN>;
  static bool once = ((void)hipFuncSetAttribute(
                          reinterpret_cast<const void*>(tiled_gemm_kernel<TM, TN, WM, WN>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS),
                      true);
  (void)once;
  const int64_t nbm = (M + G::BM - 1) / G::BM, nbn = (N + G::BN - 1) / G::BN;
  hipLaunchKernelGGL((tiled_gemm_kernel<TM, TN, WM, WN>), dim3((unsigned)(nbm * nbn)), dim3(256),
                     G::LDS, s, Xq, xs, rs, M, Kp, Wp, ws, N, Y, acc_out, (int)nbm);
  return hipGetLastError();
}

hipError_t launch_mfma32(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                         int64_t K, const uint32_t* Wp, const float* ws, int64_t N, float* Y,
                         int32_t* acc_out, hipStream_t s) {
  const int64_t Kp = (K + 63) / 64 * 64;
  // 128 x 128 tiles while those fill the CUs at most once, 128 x 256 above
  // (same box, events: 2560 -> 6912 at 256 / 512 tokens 18.1 / 19.2 against
  // 20.7 / 21.3 us, 6912 -> 2560 at 768 / 1024 / 1536 tokens 33.7 / 33.6 /
  // 35.6 against 43.5 / 43.3 / 43.9 us; 2560 -> 6912 at 768 / 1024 tokens,
  // 324 / 432 tiles of 128 x 128, 25.5 / 27.6 against 22.9 / 25.3 us)
  if (((M + 127) / 128) * ((N + 127) / 128) <= 256)
    return tiled_go<4, 1, 1, 4>(Xq, xs, rs, M, Kp, Wp, ws, N, Y, acc_out, s);
  return tiled_go<4, 2, 1, 4>(Xq, xs, rs, M, Kp, Wp, ws, N, Y, acc_out, s);
}

// The FFN's gate/up past 192 tokens on the tiled GEMM: 128 x 128 tiles of
// both matrices (the register count of one matrix's 128 x 256 tile).
hipError_t launch_tiled_gateup(const int8_t* Xq, const float* xs, const int32_t* rs, int64_t M,
                               int64_t K, const uint32_t* Wg, const float* sg, const uint32_t* Wu,
                               const float* su, int64_t N, float* H, float* gh_parts, int* nparts,
                               hipStream_t s) {
  constexpr int TM = 4, TN = 1, WM = 1, WN = 4;
  using G = TiledGemm<TM, TN, WM, WN, 2>;
  static bool once = ((void)hipFuncSetAttribute(
                          reinterpret_cast<const void*>(tiled_gemm_kernel<TM, TN, WM, WN, 2, 2>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS),
                      true);
  (void)once;
  const int64_t Kp = (K + 63) / 64 * 64;
  const int64_t nbm = (M + G::BM - 1) / G::BM, nbn = (N + G::BN - 1) / G::BN;
  if (nparts) *nparts = (int)nbn;
  hipLaunchKernelGGL((tiled_gemm_kernel<TM, TN, WM, WN, 2, 2>), dim3((unsigned)(nbm * nbn)),
                     dim3(256), G::LDS, s, Xq, xs, rs, M, Kp, Wg, sg, N, H, nullptr, (int)nbm, Wu,
                     su, gh_parts);
  return hipGetLastError();
}

}  // namespace bl

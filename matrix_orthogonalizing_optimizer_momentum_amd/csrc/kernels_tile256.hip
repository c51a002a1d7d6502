// Fused Newton-Schulz for Hierarchical-Muon tiles of side 128 < T <= 256
// (gfx950).
//
// "Hierarchical Muon: Tiled Newton-Schulz Updates for Efficient Muon
// Optimization" (core claim, abstract): every T x T tile of a momentum matrix
// gets the same finite Newton-Schulz map on its own.  Here one workgroup of
// four waves (one per SIMD, one workgroup per CU, looping over tiles) owns
// one tile at a time, zero-padded to 256 x 256 (exact: [[X, 0], [0, 0]] maps
// to [[NS(X), 0], [0, 0]]), for the whole step:
//   - momentum M <- beta M + G (Muon explainer, momentum recap / Equation 1)
//     on the tile's elements, M stored back, X0 = M and its Frobenius norm;
//   - K iterations A = X X^T; B = b A + c A A; X = a X + B X (Muon explainer,
//     Newton-Schulz section, Equation 6 and code section) with bf16 MFMA
//     operands and fp32 accumulation, 1 / (||X0|| + eps) folded into the
//     first iteration, X rounded to bf16 after every update (the FOLD
//     precision), all of it on chip;
//   - the cropped tile written once as O, with ||O||^2 and, for the weight
//     update hook, <W, O> and ||W||^2 summed where O is stored.
//
// Registers.  Wave w owns the 128 x 128 quadrant (128 (w / 2), 128 (w % 2))
// of every product: 4 x 4 accumulator blocks of 32 x 32 (256 fp32 values per
// lane), and the same quadrant of X in bf16 pairs (128 registers per lane),
// which carries X from one iteration to the next.
//
// LDS (160 KiB = one bf16 256 x 256 matrix + two 16 KiB pieces):
//   - the matrix region holds X^T for G1 (A = X X^T, read with the
//     transposing LDS read ds_read_b64_tr_b16), then A, then B (both
//     symmetric, stored from the accumulators through the transposed path),
//     and the staging of the input and output tiles; rows of 512 B, 16-byte
//     granules XOR-swizzled by the row, so that the fragment reads of 32 rows
//     at one k hit distinct banks;
//   - G3 (B X) takes X from the pieces: 32-deep slices of X^T ([n][k] rows of
//     64 B) written from the registers of the waves that hold them while
//     every wave runs the previous slice's MFMAs (double buffered).
#include <atomic>
#include <type_traits>

#include "common.h"

namespace muonh {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kS = 256;                     // padded tile side
constexpr int kNT = 256;                    // threads: 4 waves
constexpr int kMatB = kS * kS * 2;          // bytes of the bf16 matrix region
constexpr int kPieceB = 16384;              // bytes of one 32-deep X^T slice
constexpr int kSmem = kMatB + 2 * kPieceB;  // 160 KiB

// Byte offset of element (r, c) of the matrix region.
__device__ __forceinline__ int mat_off(int r, int c) {
  return r * 512 + ((((c >> 3) ^ (r & 15))) << 4) + ((c & 7) << 1);
}
// G3 slice: X^T(n, k0 + kk) for kk < 32, rows n of 64 B, granules swizzled by
// n / 4 so that 16 consecutive rows read at one kk hit 16 distinct granules.
__device__ __forceinline__ int g3_off(int n, int kk) {
  return n * 64 + ((((kk >> 3) ^ ((n >> 2) & 3))) << 4) + ((kk & 7) << 1);
}
// X^T for G1 in the matrix region: element (n, m) in row n (512 B), column
// (m + 32 (n % 4)) % 256, whose 16-byte granule is XORed with (n / 4) % 4.
// The rotation puts the four rows one transposing read touches in different
// banks; the XOR (the same for those four rows) spreads the 8-byte writes of
// 32 consecutive rows.
__device__ __forceinline__ int xt_off(int n, int m) {
  const int rot = (m + 32 * (n & 3)) & 255;
  return n * 512 + ((((rot >> 3) ^ ((n >> 2) & 3))) << 4) + ((rot & 7) << 1);
}

template <typename P>
__device__ __forceinline__ __attribute__((address_space(3))) P* lds(void* p) {
  return (__attribute__((address_space(3))) P*)p;
}

__device__ __forceinline__ bf16x8_t ld16(const char* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// Transposing read pair: one MFMA operand fragment (8 consecutive k of one
// row m) from a [k][m] slice, as in the GEMM engine.
__device__ __forceinline__ bf16x8_t ld_tr8(const char* p0, const char* p1) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds<i16x4_t>(const_cast<char*>(p0)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds<i16x4_t>(const_cast<char*>(p1)));
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N - 1>{})
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// The LDS addresses below depend only on the lane and compile-time offsets,
// so the compiler would hoist every one of them out of the iteration loop and
// spill them; passing the lane base through an empty asm per use keeps them
// computed where they are used.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// wave_sum with the lane id passed in (the same exchanges and additions, so
// the same bits): the lane addresses are then not loop invariant either.
__device__ __forceinline__ double wave_sum_at(double v, int lane) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int a = (lane ^ o) << 2;
    const int lo = __builtin_amdgcn_ds_bpermute(a, __double2loint(v));
    const int hi = __builtin_amdgcn_ds_bpermute(a, __double2hiint(v));
    v += __hiloint2double(hi, lo);
  }
  return v;
}

__device__ __forceinline__ float lo_bf(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

}  // namespace

// One tile, start to end (the caller's barrier separates it from the
// workgroup's previous tile).
__device__ __forceinline__ void tile256_one(char* const smem, const TileMat* __restrict__ mats, const TileJob job,
                                            const TileArgs& args, const int tid) {
  char* const sM = smem;
  char* const sP0 = smem + kMatB;
  // reduction scratch in the second slice: it is first written by G3 of the
  // first iteration, long after every thread's read of the pre-scale sum
  double* const sred = reinterpret_cast<double*>(smem + kMatB + kPieceB);

  const TileMat mt = mats[job.mat];
  const int T = args.T;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = (wave >> 1) * 128, wc = (wave & 1) * 128;  // quadrant origin
  const int lc = lane & 31, lh = lane >> 5;
  const int64_t r0 = (int64_t)job.ti * T, c0 = (int64_t)job.tj * T;
  const int h = (int)min<int64_t>(T, mt.H - r0), w = (int)min<int64_t>(T, mt.W - c0);
  const int64_t ldm = mt.W;
  const bf16_t* const tg = mt.g ? reinterpret_cast<const bf16_t*>(mt.g) + r0 * ldm + c0 : nullptr;
  bf16_t* const tm = reinterpret_cast<bf16_t*>(mt.m) + r0 * ldm + c0;

  // ---- input: momentum on the tile (8-element row chunks, chunk t + 256 c
  // for thread t), M stored back, X0 staged row-major in the matrix region.
  float sq = 0.f;
  if (mt.vec) {
    // batches of 8 chunks of M (and G), three batches in flight: with one
    // workgroup per CU the loads must cover HBM latency on their own, so the
    // next batch is issued as soon as one has been consumed
    u32x4_t mraw[3][8], graw[3][8];
    auto load_in = [&](int cb, u32x4_t (&mr)[8], u32x4_t (&gr)[8]) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = 8 * (cb + k) + (tid >> 5), col = (tid & 31) * 8;
        const int64_t off = (row < h && col < w) ? (int64_t)row * ldm + col : 0;
        mr[k] = *reinterpret_cast<const MUONH_GLOBAL u32x4_t*>(gmem(tm + off));
        if (tg) gr[k] = *reinterpret_cast<const MUONH_GLOBAL u32x4_t*>(gmem(tg + off));
      }
    };
    load_in(0, mraw[0], graw[0]);
    load_in(8, mraw[1], graw[1]);
    load_in(16, mraw[2], graw[2]);
    static_for<4>([&](auto bc) {
      constexpr int bi = decltype(bc)::value, cb = 8 * bi, sl = bi % 3;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = 8 * (cb + k) + (tid >> 5), col = (tid & 31) * 8;
        const bool ok = row < h && col < w;
        u32x4_t pk = mraw[sl][k];
        if (tg) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[2 * e] = St<bf16_t>::round(fmaf(args.beta, lo_bf(mraw[sl][k][e]), args.gcoef * lo_bf(graw[sl][k][e])));
            x[2 * e + 1] = St<bf16_t>::round(fmaf(args.beta, hi_bf(mraw[sl][k][e]), args.gcoef * hi_bf(graw[sl][k][e])));
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
          if (ok) *reinterpret_cast<MUONH_GLOBAL u32x4_t*>(gmem(tm + (int64_t)row * ldm + col)) = pk;
        }
        if (!ok) pk = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sq = fmaf(lo_bf(pk[e]), lo_bf(pk[e]), sq);
          sq = fmaf(hi_bf(pk[e]), hi_bf(pk[e]), sq);
        }
        *reinterpret_cast<u32x4_t*>(sM + mat_off(row, col)) = pk;
      }
      if constexpr (bi == 0) load_in(24, mraw[0], graw[0]);
    });
  } else {
#pragma unroll 1
    for (int c = 0; c < 32; ++c) {
      const int row = 8 * c + (tid >> 5), col = (tid & 31) * 8;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float v = 0.f;
        if (row < h && col + e < w) {
          const int64_t o = (int64_t)row * ldm + col + e;
          v = St<bf16_t>::ld(tm, o);
          if (tg) {
            v = St<bf16_t>::round(fmaf(args.beta, v, args.gcoef * St<bf16_t>::ld(tg, o)));
            St<bf16_t>::st(tm, o, v);
          }
        }
        x[e] = v;
        sq = fmaf(v, v, sq);
      }
      u32x4_t pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(x[2 * e], x[2 * e + 1]);
      *reinterpret_cast<u32x4_t*>(sM + mat_off(row, col)) = pk;
    }
  }
  {
    const double d = wave_sum_at((double)sq, lane);
    if (lane == 0) sred[wave] = d;
  }
  __syncthreads();
  // (eps through the empty asm: its fp64 conversion is not held across tiles)
  const double sig =
      1.0 / (sqrt(((sred[0] + sred[1]) + sred[2]) + sred[3]) + (double)__int_as_float(opaque(__float_as_int(args.eps))));

  // X0 into registers in the accumulator layout: lane l of block (i, j),
  // group q holds rows 8 q + 4 (l / 32) + 0..3 of column l % 32 -- one
  // transposing read of the row-major staging per group (16-lane group g
  // reads the 4 x 16 block at rows + 4 (g / 2), columns + 16 (g % 2)).
  u32x2_t xr[4][4][4];  // bf16 pairs: rows (0, 1) and (2, 3) of a group
  {
    const int j16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int R = wr + i * 32 + 8 * q + 4 * (g >> 1) + (j16 >> 2);
          const int C = wc + j * 32 + 16 * (g & 1) + 4 * (j16 & 3);
          const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds<i16x4_t>(sM + mat_off(R, C)));
          xr[i][j][q] = __builtin_bit_cast(u32x2_t, v);
        }
  }
  // every wave has its X0 before the first iteration writes X^T over the
  // staging (a wave's quadrant of X^T covers rows another wave gathers from)
  __syncthreads();

  // Accumulators are written only by MFMAs: the first k-step of a product
  // takes a zero C operand, and the seed terms (b A, a X) are added in the
  // epilogues, which only read them.  (Element writes into the accumulator
  // tuples between products make the compiler move whole tuples through the
  // arch VGPRs, which then spill.)
  f32x16_t acc[4][4];
  // 16 MFMAs of the wave's quadrant, calling next(i) after the four that
  // read fa[i] have issued (a load into fa[i] may follow them)
  auto mma16_next = [&](bf16x8_t (&fa)[4], const bf16x8_t (&fb)[4], auto zc, auto next) {
    constexpr bool zero = decltype(zc)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], zero ? f32x16_t{} : acc[i][j], 0, 0, 0);
      next(i);
    }
  };
  using Z = std::true_type;
  using NZ = std::false_type;
  auto bar = [] {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };

  // G3 slice p: X^T(n, 32 p + kk), written by the two waves whose row range
  // holds rows 32 p .. 32 p + 31 of X (their block row p % 4).  The slice
  // loop is unrolled, so p (and the register block) is a compile-time
  // constant: indexing the register array at run time would move it to
  // scratch memory.  Slice element (n, 8 q + 4 lh), n = wc + 32 j + lc, is
  // at row n, granule q ^ (lc / 4 % 4); every lane base is derived from a
  // fresh opaque copy of the lane id where it is used.
  //
  // G1 reads X^T whole from the matrix region (free at that point): every
  // wave writes its quadrant, X(m..m+3, n) -> X^T(n, m..m+3).
  auto put_xt = [&]() {
    const int ln = opaque(lane), l31 = ln & 31, lhh = ln >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<u32x2_t*>(sM + xt_off(wc + 32 * j + l31, wr + 32 * i + 8 * q + 4 * lhh)) = xr[i][j][q];
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  auto put_g3 = [&](auto pc, char* buf) {
    constexpr int p = decltype(pc)::value, ib = p & 3;
    if ((p >> 2) != (wave >> 1)) return;  // uniform per wave
    const int ln = opaque(lane), l31 = ln & 31;
    const int base = (wc + l31) * 64 + 8 * (ln >> 5), sw = (l31 >> 2) & 3;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      char* const bq = buf + base + ((q ^ sw) << 4);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<u32x2_t*>(bq + 2048 * j) = xr[ib][j][q];
    }
  };

  // ---- The symmetric products A = X X^T and A A on their distinct blocks
  // only.  In 32-row blocks of the 256 x 256 matrix, waves 0 and 1 each take
  // half of the upper right quadrant (blocks I = 0..3 by J = 4 + 2 w, 5 + 2 w,
  // from fragments of 4 row blocks and 2 column blocks) plus one block those
  // fragments also give, (4, 5) for wave 0 and (0, 1) for wave 1; waves 2 and
  // 3 the other blocks I <= J of the upper left / lower right quadrant (P and
  // Q are the same matrix, so the fragments of its 4 blocks serve every one
  // of them): 36 of the 64 blocks, 9 per wave against 16.  A wave stores its blocks through the transposed path (block
  // (I, J) lands at (J, I), in the lower triangle: for a symmetric result the
  // cheap 8-byte writes of the accumulator layout).  G2 reads A from there,
  // the part above the diagonal through transposing reads; B is copied into
  // its upper positions as well (transposing reads again), so that G3 reads
  // whole rows.
  const int qb = 4 * (wave & 1);      // tri waves: first block of the quadrant
  const int cbk = 4 + 2 * (wave & 1);  // rect waves: first column block
  // The accumulator slots of a wave, 9 each: tri: acc[i][j], j >= i, except
  // (0, 1) = block (qb + i, qb + j); rect: acc[i][j], j < 2 = block
  // (i, cbk + j), and acc[0][2] = the extra block, (cbk, cbk + 1) for wave 0
  // and (0, 1) for wave 1.
  auto slot_ok = [](bool TRI, int i, int j) {
    return TRI ? (j >= i && !(i == 0 && j == 1)) : (j < 2 || (i == 0 && j == 2));
  };
  auto blk_i = [&](auto tri_c, int i, int j) {
    return decltype(tri_c)::value ? qb + i : j < 2 ? i : (wave & 1) ? 0 : cbk;
  };
  auto blk_j = [&](auto tri_c, int i, int j) {
    return decltype(tri_c)::value ? qb + j : j < 2 ? cbk + j : (wave & 1) ? 1 : cbk + 1;
  };
  // fragment f of a wave: tri: block qb + f; rect: blocks 0..3, then cbk, cbk + 1
  auto frag_blk = [&](auto tri_c, int f) { return decltype(tri_c)::value ? qb + f : (f < 4 ? f : cbk + f - 4); };

  // G1 (g1 true: transposing reads of X^T, k = n) or G2 (plain reads of A
  // rows) over the wave's blocks.  G1 fragments: lane 16 g + j16 reads rows
  // 16 ks + 8 (g / 2) + j16 / 4 and 4 rows further, elements 16 (g % 2) +
  // 4 (j16 % 4) of its 32-wide block (the layout repeats every 16 rows, so a
  // k-step adds 8 KiB; the two reads differ in their granule XOR).  G2
  // fragments: row 32 X + lc, granule (2 ks + lh) ^ (lc % 16).
  auto sym_product = [&](auto tri_c, auto g1_c, auto w1_c) __attribute__((always_inline)) {
    constexpr bool TRI = decltype(tri_c)::value;
    constexpr bool G1 = decltype(g1_c)::value;
    // G2 of a wave whose blocks are known at compile time (w1_c: wave % 2)
    // reads A from its lower triangle only: for k in a block K above the
    // fragment's block X, A(32 X + lc, k) = A(k, 32 X + lc) comes from the
    // stored block (K, X) through transposing reads (as G1 reads X^T)
    constexpr int W1 = decltype(w1_c)::value;  // -1: not specialised
    constexpr bool LOWER = !G1 && W1 >= 0;
    constexpr int NF = TRI ? 4 : 6;
    auto fblk_ct = [](int f) { return TRI ? 4 * W1 + f : (f < 4 ? f : 4 + 2 * W1 + f - 4); };
    int off[2][NF], tro[2][NF];
    {
      const int ln = opaque(lane);
      const int j16 = ln & 15, g = ln >> 4;
      const int krow = 8 * (g >> 1) + (j16 >> 2), msub = 16 * (g & 1) + 4 * (j16 & 3);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int X = LOWER ? fblk_ct(f) : frag_blk(tri_c, f);
        if constexpr (G1) {
          off[0][f] = xt_off(krow, 32 * X + msub);
          off[1][f] = xt_off(krow + 4, 32 * X + msub);
        } else {
          off[0][f] = (32 * X + (ln & 31)) * 512;
          off[1][f] = 0;
          if constexpr (LOWER) {
            // rows 16 ks + krow (+ 4): the granule XOR depends on the row
            // modulo 16 only, so a k-step adds 8 KiB
            tro[0][f] = mat_off(krow, 32 * X + msub);
            tro[1][f] = mat_off(krow + 4, 32 * X + msub);
          }
        }
      }
    }
    bf16x8_t fr[2][NF];
    auto ld = [&](int buf, auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      if constexpr (G1) {
        constexpr int o = ks * 16 * 512;  // 16 rows further
#pragma unroll
        for (int f = 0; f < NF; ++f) fr[buf][f] = ld_tr8(sM + off[0][f] + o, sM + off[1][f] + o);
      } else {
        const int ln = opaque(lane);
        const int gofs = ((2 * ks + (ln >> 5)) ^ (ln & 15)) << 4;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (LOWER && ks / 2 > fblk_ct(f))
            fr[buf][f] = ld_tr8(sM + tro[0][f] + ks * 8192, sM + tro[1][f] + ks * 8192);
          else
            fr[buf][f] = ld16(sM + off[0][f] + gofs);
        }
      }
    };
    auto mm = [&](int buf, auto zc) {
      constexpr bool zero = decltype(zc)::value;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (!slot_ok(TRI, i, j)) continue;
          bf16x8_t fp = fr[buf][i], fq = TRI ? fr[buf][j] : fr[buf][4 + (j & 1)];
          if (!TRI && j == 2) {
            // the extra block: fragments 4, 5 (wave 0) or 0, 1 (wave 1)
            const bool w1 = W1 >= 0 ? W1 == 1 : (wave & 1) != 0;
            fp = w1 ? fr[buf][0] : fr[buf][4];
            fq = w1 ? fr[buf][1] : fr[buf][5];
          }
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp, fq, zero ? f32x16_t{} : acc[i][j], 0, 0, 0);
        }
    };
    ld(0, std::integral_constant<int, 0>{});
    static_for<8>([&](auto hc) {
      constexpr int ks = 2 * decltype(hc)::value;
      ld(1, std::integral_constant<int, ks + 1>{});
      __builtin_amdgcn_sched_barrier(0);
      mm(0, std::integral_constant<bool, ks == 0>{});
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (ks + 2 < 16) ld(0, std::integral_constant<int, ks + 2>{});
      __builtin_amdgcn_sched_barrier(0);
      mm(1, NZ{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // Element group q of the lane's value of block (I, J) -- rows 32 I + 8 q +
  // 4 lh + 0..3 of column 32 J + lc -- goes to row 32 J + lc, elements
  // 32 I + 8 q + 4 lh.. (mat_off: granule (4 I + q) ^ (lc % 16), byte 8 lh).
  // (lb: the lane's part, 512 lc + 8 lh and lc % 16, derived once per pass)
  struct LaneBase {
    int row, sw;
  };
  auto lane_base = [&]() {
    const int ln = opaque(lane), l31 = ln & 31;
    return LaneBase{l31 * 512 + 8 * (ln >> 5), l31 & 15};
  };
  auto lo_addr = [&](const LaneBase& lb, int I, int J, int q) -> char* {
    return sM + lb.row + 16384 * J + (((4 * I + q) ^ lb.sw) << 4);
  };
  // A = sc * acc (scaled: times sc, the first iteration's sig^2 and 1 after
  // it; a run-time branch between the two forms would join register states)
  auto put_a = [&](auto tri_c, auto scaled, float sc) __attribute__((always_inline)) {
    constexpr bool TRI = decltype(tri_c)::value;
    constexpr bool kScale = decltype(scaled)::value;
    const LaneBase lb = lane_base();
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!slot_ok(TRI, i, j)) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = kScale ? acc[i][j][4 * q + e] * sc : acc[i][j][4 * q + e];
          *reinterpret_cast<u32x2_t*>(lo_addr(lb, blk_i(tri_c, i, j), blk_j(tri_c, i, j), q)) =
              u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
        // one block at a time: the scheduler would otherwise batch every
        // accumulator read (register pressure)
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // B = c * acc + b * A, with A read back from the very slot the lane then
  // overwrites (c = 0: B = b A, acc unused); the next block's four A reads
  // are in flight while this block is formed
  auto put_b = [&](auto tri_c, float b, float c) __attribute__((always_inline)) {
    constexpr bool TRI = decltype(tri_c)::value;
    constexpr int NB = 9;
    // slot t of the wave in order
    constexpr int kTi[9] = {0, 0, 0, 1, 1, 1, 2, 2, 3}, kTj[9] = {0, 2, 3, 1, 2, 3, 2, 3, 3};
    constexpr int kRi[9] = {0, 0, 1, 1, 2, 2, 3, 3, 0}, kRj[9] = {0, 1, 0, 1, 0, 1, 0, 1, 2};
    auto bi = [&](int t) { return TRI ? kTi[t] : kRi[t]; };
    auto bj = [&](int t) { return TRI ? kTj[t] : kRj[t]; };
    const LaneBase lb = lane_base();
    u32x2_t av[2][4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      av[0][q] = *reinterpret_cast<const u32x2_t*>(lo_addr(lb, blk_i(tri_c, bi(0), bj(0)), blk_j(tri_c, bi(0), bj(0)), q));
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int i = bi(t), j = bj(t), cur = t & 1;
      if (t + 1 < NB) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          av[cur ^ 1][q] = *reinterpret_cast<const u32x2_t*>(
              lo_addr(lb, blk_i(tri_c, bi(t + 1), bj(t + 1)), blk_j(tri_c, bi(t + 1), bj(t + 1)), q));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2_t a2 = av[cur][q];
        float v[4] = {b * lo_bf(a2[0]), b * hi_bf(a2[0]), b * lo_bf(a2[1]), b * hi_bf(a2[1])};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = fmaf(c, acc[i][j][4 * q + e], v[e]);
        *reinterpret_cast<u32x2_t*>(lo_addr(lb, blk_i(tri_c, i, j), blk_j(tri_c, i, j), q)) =
            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The wave's own blocks above the diagonal (I < J), each from its mirror
  // (J, I) that the wave has just stored below it: a transposing read gives
  // the lane rows 32 J + 8 q + 4 lh + 0..3 of column 32 I + lc, which are
  // elements 32 J + 8 q + 4 lh.. of row 32 I + lc, one 8-byte write.  A
  // wave's LDS accesses run in order, so it needs no barrier to read back its
  // own stores; all reads are issued before the first write.
  auto mirror = [&](auto tri_c) __attribute__((always_inline)) {
    constexpr bool TRI = decltype(tri_c)::value;
    constexpr int NM = TRI ? 5 : 9;
    // slot t of the wave off the diagonal: tri (i, j) with i < j but (0, 1),
    // rect all
    constexpr int kTi[5] = {0, 0, 1, 1, 2}, kTj[5] = {2, 3, 2, 3, 3};
    constexpr int kRi[9] = {0, 0, 1, 1, 2, 2, 3, 3, 0}, kRj[9] = {0, 1, 0, 1, 0, 1, 0, 1, 2};
    auto mi = [&](int t) { return TRI ? kTi[t] : kRi[t]; };
    auto mj = [&](int t) { return TRI ? kTj[t] : kRj[t]; };
    const int ln = opaque(lane), j16 = ln & 15, g = ln >> 4;
    u32x2_t v[NM][4];
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      const int I = blk_i(tri_c, mi(t), mj(t)), J = blk_j(tri_c, mi(t), mj(t));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int R = 32 * J + 8 * q + 4 * (g >> 1) + (j16 >> 2);
        const int C = 32 * I + 16 * (g & 1) + 4 * (j16 & 3);
        v[t][q] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds<i16x4_t>(sM + mat_off(R, C))));
      }
    }
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      const int I = blk_i(tri_c, mi(t), mj(t)), J = blk_j(tri_c, mi(t), mj(t));
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x2_t*>(sM + mat_off(32 * I + (ln & 31), 32 * J + 8 * q + 4 * (ln >> 5))) = v[t][q];
    }
  };
  const bool tri = (wave & 2) != 0;
  using TRI_T = std::true_type;
  using RECT_T = std::false_type;

  for (int it = 0; it < args.K; ++it) {
    const float a = args.abc[it][0], b = args.abc[it][1], c = args.abc[it][2];
    const bool first = it == 0;

    // ---------------- G1: A = X X^T (times sig^2 on the first iteration),
    // stored below the diagonal; the product and the store stay inside one
    // wave-uniform branch, so no accumulator state is live where the two
    // paths join.  G2 (A A) runs for c = 0 too (c * A A then adds nothing): a
    // run-time branch around it would join two accumulator states, which the
    // compiler resolves by copying all of them through the arch VGPRs.
    put_xt();
    bar();
    const float asc = first ? (float)(sig * sig) : 1.f;  // branch-free (see update below)
    using ANY = std::integral_constant<int, -1>;
    if (tri) {
      sym_product(TRI_T{}, std::true_type{}, ANY{});
      bar();  // every wave is done reading X^T
      put_a(TRI_T{}, std::true_type{}, asc);
    } else {
      sym_product(RECT_T{}, std::true_type{}, ANY{});
      bar();
      put_a(RECT_T{}, std::true_type{}, asc);
    }
    bar();

    // ---------------- G2: B = b A + c A A, stored below the diagonal, then
    // mirrored (on the first iteration B is stored times sig, which with
    // a * sig in the update gives sig (a X0 + B X0) without scaling the
    // accumulators)
    const float xs = first ? (float)sig : 1.f;
    // (A is only below the diagonal: G2 reads the rest transposed, which
    // needs the wave's blocks at compile time)
    auto g2 = [&](auto tri_c, auto w1_c) __attribute__((always_inline)) {
      sym_product(tri_c, std::false_type{}, w1_c);
      bar();  // every wave is done reading A
      put_b(tri_c, b * xs, c * xs);
      mirror(tri_c);
    };
    using W0 = std::integral_constant<int, 0>;
    using W1 = std::integral_constant<int, 1>;
    if (wave == 3) g2(TRI_T{}, W1{});
    else if (wave == 2) g2(TRI_T{}, W0{});
    else if (wave == 1) g2(RECT_T{}, W1{});
    else g2(RECT_T{}, W0{});

    // ---------------- G3: X <- a X + B X (times sig on the first)
    put_g3(std::integral_constant<int, 0>{}, sP0);
    bar();
    {
      // B rows wr + 32 i + lc at k = 32 p + 16 kk + 8 lh (the A operand) do
      // not change during G3: each slice's are loaded during the previous
      // slice's MFMAs, row block i as soon as the MFMAs that read the old
      // fragment i have issued; after the barrier only the slice's own
      // fragments (rows wc + 32 j + lc at kk16 = 16 kk + 8 lh) are read.
      bf16x8_t fa[2][4], fb[2][4];
      auto ld_brow = [&](int p, int kk, int i) {
        const int ln = opaque(lane), l31 = ln & 31, lhh = ln >> 5;
        fa[kk][i] = ld16(sM + (wr + l31) * 512 + (((4 * p + 2 * kk + lhh) ^ (l31 & 15)) << 4) + 16384 * i);
      };
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) ld_brow(0, kk, i);
      static_for<8>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int so = (p & 1) * kPieceB;  // this slice's buffer
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const int ln = opaque(lane), l31 = ln & 31, lhh = ln >> 5;
          const char* pb = smem + so + kMatB + (wc + l31) * 64 + (((2 * kk + lhh) ^ ((l31 >> 2) & 3)) << 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) fb[kk][j] = ld16(pb + 2048 * j);
        }
        __builtin_amdgcn_sched_barrier(0);
        mma16_next(fa[0], fb[0], std::integral_constant<bool, p == 0>{}, [&](int i) {
          if constexpr (p + 1 < 8) ld_brow(p + 1, 0, i);
        });
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (p + 1 < 8) put_g3(std::integral_constant<int, p + 1>{}, sP0 + ((p + 1) & 1) * kPieceB);
        __builtin_amdgcn_sched_barrier(0);
        mma16_next(fa[1], fb[1], NZ{}, [&](int i) {
          if constexpr (p + 1 < 8) ld_brow(p + 1, 1, i);
        });
        bar();
      });
    }
    // X <- (a sig) X + (sig B) X on the first iteration, a X + B X after it,
    // rounded to bf16 and kept in registers for the next iteration
    {
      const float ax = a * xs;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t x0 = xr[i][j][q][0], x1 = xr[i][j][q][1];
            const float v[4] = {fmaf(ax, lo_bf(x0), acc[i][j][4 * q]), fmaf(ax, hi_bf(x0), acc[i][j][4 * q + 1]),
                                fmaf(ax, lo_bf(x1), acc[i][j][4 * q + 2]), fmaf(ax, hi_bf(x1), acc[i][j][4 * q + 3])};
            xr[i][j][q] = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            if (q == 3) __builtin_amdgcn_sched_barrier(0);
          }
    }
  }
  if (args.K == 0) {  // O = X0 / (||X0|| + eps)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t w0 = xr[i][j][q][0], w1 = xr[i][j][q][1];
          xr[i][j][q] = u32x2_t{pack_bf16x2((float)((double)lo_bf(w0) * sig), (float)((double)hi_bf(w0) * sig)),
                                pack_bf16x2((float)((double)lo_bf(w1) * sig), (float)((double)hi_bf(w1) * sig))};
        }
  }

  // ---- output: O (bf16) staged row-major in the matrix region (behind a
  // barrier: the last product's reads, or with K = 0 the X0 gather), then written as
  // 8-element row chunks cropped to the matrix, with ||O||^2 and the hook's
  // <W, O>, ||W||^2 at the same positions (fp64 per thread).  The W rows do
  // not depend on the result: the first batch is loaded before the staging,
  // and each later one while the previous batch is consumed.
  const float* const wp = mt.w;
  const int64_t obase = r0 * ldm + c0;
  typedef __attribute__((address_space(4))) const f32x4_t cf4;
  f32x4_t wv[2][8][2];
  auto load_w = [&](int cb, f32x4_t (&d)[8][2]) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int row = 8 * (cb + k) + (tid >> 5), col = (tid & 31) * 8;
      const int64_t o = (row < h && col < w) ? obase + (int64_t)row * ldm + col : obase;
      d[k][0] = *reinterpret_cast<cf4*>(reinterpret_cast<uintptr_t>(wp + o));
      d[k][1] = *reinterpret_cast<cf4*>(reinterpret_cast<uintptr_t>(wp + o + 4));
    }
  };
  if (mt.vec && wp != nullptr) load_w(0, wv[0]);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = wr + i * 32 + 8 * q + 4 * lh, n = wc + j * 32 + lc;
        const uint32_t w0 = xr[i][j][q][0], w1 = xr[i][j][q][1];
        *reinterpret_cast<bf16_t*>(sM + mat_off(m + 0, n)) = (bf16_t)(w0 & 0xffffu);
        *reinterpret_cast<bf16_t*>(sM + mat_off(m + 1, n)) = (bf16_t)(w0 >> 16);
        *reinterpret_cast<bf16_t*>(sM + mat_off(m + 2, n)) = (bf16_t)(w1 & 0xffffu);
        *reinterpret_cast<bf16_t*>(sM + mat_off(m + 3, n)) = (bf16_t)(w1 >> 16);
      }
  __syncthreads();
  double osq = 0.0, swo = 0.0, sww = 0.0;
  if (mt.vec) {
    static_for<4>([&](auto bc) {
      constexpr int bi = decltype(bc)::value, cb = 8 * bi, sl = bi & 1;
      if constexpr (bi < 3) {
        if (wp != nullptr) load_w(cb + 8, wv[sl ^ 1]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = 8 * (cb + k) + (tid >> 5), col = (tid & 31) * 8;
        if (row >= h || col >= w) continue;
        const u32x4_t pk = *reinterpret_cast<const u32x4_t*>(sM + mat_off(row, col));
        const int64_t o = obase + (int64_t)row * ldm + col;
        *reinterpret_cast<MUONH_GLOBAL u32x4_t*>(gmem(reinterpret_cast<bf16_t*>(mt.out) + o)) = pk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const double x = (double)((e & 1) ? hi_bf(pk[e >> 1]) : lo_bf(pk[e >> 1]));
          osq = fma(x, x, osq);
          if (wp != nullptr) {
            const double wd = (double)wv[sl][k][e >> 2][e & 3];
            swo = fma(wd, x, swo);
            sww = fma(wd, wd, sww);
          }
        }
      }
    });
  } else {
#pragma unroll 1
    for (int cch = 0; cch < 32; ++cch) {
      const int row = 8 * cch + (tid >> 5), col = (tid & 31) * 8;
      if (row >= h || col >= w) continue;
      const u32x4_t pk = *reinterpret_cast<const u32x4_t*>(sM + mat_off(row, col));
      const int64_t o = obase + (int64_t)row * ldm + col;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < w) {
          const float x = (e & 1) ? hi_bf(pk[e >> 1]) : lo_bf(pk[e >> 1]);
          store_dyn(mt.out, o + e, x, DT_BF16);
          osq = fma((double)x, (double)x, osq);
          if (wp != nullptr) {
            const double wd = (double)load1_ro(wp, o + e);
            swo = fma(wd, (double)x, swo);
            sww = fma(wd, wd, sww);
          }
        }
    }
  }
  // block sums: one fp64 partial per tile (the slices are idle: scratch)
  {
    const int ln = opaque(lane);  // (lane addresses derived here, not shared with the input's sum)
    osq = wave_sum_at(osq, ln);
    swo = wave_sum_at(swo, ln);
    sww = wave_sum_at(sww, ln);
  }
  if (lane == 0) {
    sred[wave] = osq;
    sred[4 + wave] = swo;
    sred[8 + wave] = sww;
  }
  __syncthreads();
  if (tid == 0) {
    const double t0 = ((sred[0] + sred[1]) + sred[2]) + sred[3];
    const double t1 = ((sred[4] + sred[5]) + sred[6]) + sred[7];
    const double t2 = ((sred[8] + sred[9]) + sred[10]) + sred[11];
    const SlotTable& st = args.st;
    const int64_t pa = st.part_base[mt.onorm_slot] + job.part;
    gmem(st.partials)[2 * pa] = t0;
    gmem(st.partials)[2 * pa + 1] = wp != nullptr ? t1 : 0.0;
    if (wp != nullptr) {
      const int64_t pb = st.part_base[mt.hook_slot] + job.part;
      gmem(st.partials)[2 * pb] = 0.0;
      gmem(st.partials)[2 * pb + 1] = t2;
    }
  }
}

// Persistent: one workgroup per CU, workgroup b takes tiles b, b + grid, ...
// (with a grid of all CUs, a multiple of 8, tile j stays on XCD j % 8, as
// with one workgroup per tile).
// Every tile costs the same, so workgroups that start together stay in step
// and all of them load their inputs, and later store their outputs, at the
// same moments, sharing HBM 256 ways while its bandwidth is idle the rest of
// the tile.  With stagger > 0 the upper half of the grid first waits that
// many ticks of the 100 MHz real-time counter (about half a tile), so that
// one half's loads and stores fall into the other half's products.  The wait
// ends after at most kMaxNaps naps whatever the counter reads.
constexpr int kMaxNaps = 4096;

__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_tile256_ns(const TileMat* __restrict__ mats, const TileJob* __restrict__ jobs, int njobs, TileArgs args,
                  int stagger) {
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  if (stagger > 0 && 2 * (int)blockIdx.x >= (int)gridDim.x) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int k = 0; k < kMaxNaps && __builtin_amdgcn_s_memrealtime() - t0 < (uint64_t)stagger; ++k)
      __builtin_amdgcn_s_sleep(127);
  }
  for (int jb = blockIdx.x; jb < njobs; jb += gridDim.x) {
    __syncthreads();  // the previous tile's last LDS reads are done
    // (the thread id through an empty asm: nothing derived from it is loop
    // invariant, so nothing is held in registers across the tiles)
    tile256_one(smem, mats, jobs[jb], args, opaque((int)threadIdx.x));
  }
}

hipError_t launch_tile256_ns(const TileMat* mats, const TileJob* jobs, int njobs, const TileArgs& args,
                             hipStream_t s) {
  if (njobs <= 0) return hipSuccess;
  if (args.T <= kTileResidentMax || args.T > kTileFusedMax || args.K < 0 || args.K > kTileMaxK || !args.fold)
    return hipErrorInvalidValue;
  // one workgroup fills a CU (all of its LDS)
  static std::atomic<int> cus[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int ncu = cus[dev].load(std::memory_order_relaxed);
  if (ncu == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    ncu = n > 8 ? n / 8 * 8 : 8;
    cus[dev].store(ncu, std::memory_order_relaxed);
  }
  const int grid = njobs < ncu ? njobs : ncu;
  // Stagger only when every workgroup has two tiles or more; the extra tiles
  // of a ragged count go to the lower half, which does not wait.  The wait is
  // half a tile: about 28 us of loads and stores plus 21 us per iteration on
  // MI355X.
  const int stagger = njobs >= 2 * grid && njobs % grid <= grid / 2 ? (1400 + 1050 * args.K) : 0;
  hipLaunchKernelGGL(k_tile256_ns, dim3(grid), dim3(kNT), 0, s, mats, jobs, njobs, args, stagger);
  return hipGetLastError();
}

}  // namespace muonh

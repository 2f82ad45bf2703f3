// Quantize-append kernels for gfx950 (CDNA4): QSAC centre choice, INT2 residual
// tiles and PSAC INT8 compensation for Keys; nearest centre + INT2 for Values.
//
// Method: QuantWM ([digest] "Flickering after quantization? A temporally stable
// 2-bit KV Cache compression framework for video world models emerges", QSAC
// and PSAC paragraphs; [review] summary, Eq. 7).  The arithmetic of every
// stored field is the one documented for qwm_quantize_append_k in qwm.h.
//
// Work decomposition.  A workgroup (4 or 8 waves) serves one head; each wave
// takes two segments of <= 32 tokens (one 32-token MFMA N-block each).  The
// head's centre codebook is staged once in LDS (bf16, rows padded by 16 bytes,
// C rounded up to pairs of 32-centre blocks).
//
//  1. Screen (MFMA, bf16 -> fp32): F_c = x . mu_c - ||mu_c||_s^2 / 2 for all c,
//     x = s * k split into bf16 hi + lo (Values: x = v, exact in bf16), so
//     argmax F = argmin D.  A = 32 centres x 16 channels from LDS, B = 32
//     tokens x 16 channels from registers; the accumulator starts at
//     -||mu||_s^2/2.  Lane (t, h) ends with token t's scores of 16 centres per
//     block; it keeps the top K_c + 3 (Values: 3) as float keys whose low bits
//     carry the centre index (one and-or, L - 1 med3 and one max per score).  The
//     MFMAs of the next block run while the keys of this one are inserted.
//  2. Lane = token: v_permlane32_swap hands lane t token t of the first segment
//     and lane t + 32 token t of the second, with both halves of its list and
//     of ||k||_s^2 (and, for bf16 Values, of its row, kept from the screen).
//  3. Certification: |F~_c - F_c| <= eps_c (bound below).  If the members'
//     lower bars clear the outsiders' upper bars the candidate set is exact;
//     otherwise the uncertain entries are rescored in fp64, four (token,
//     centre) pairs at a time by the whole wave, or (rare) the wave searches
//     all centres for the token.
//  4. QSAC stage 2 scores the candidates' residual ranges in fp64 (or, for
//     the ablation scores, their one-token INT2 errors in the diagonal or the
//     full quadratic form); the INT2 tile min/max is a DPP butterfly over the
//     T lanes of a tile; PSAC accumulates c = U^T e in fp64 with U read
//     wave-uniformly from LDS, in passes of at most 16 columns.
#pragma once
#include "qwm_internal.h"

#include <hip/hip_fp16.h>

#include <algorithm>

namespace qwm {
namespace append_detail {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPad = 8;  // bf16 elements of padding per LDS codebook row

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint16_t to_half_bits(float x) {
  return __half_as_ushort(__float2half_rn(x));
}
__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// Insert a key into a descending list of L keys (keeps the L largest).
template <int L>
__device__ __forceinline__ void topl_insert(float (&l)[L], float x) {
#pragma unroll
  for (int i = L - 1; i >= 1; --i) l[i] = __builtin_amdgcn_fmed3f(l[i - 1], l[i], x);
  // max(l[0], x) for keys below +FLT_MAX, in one instruction (a med3 against
  // +inf would become a max with NaN canonicalisation of x)
  l[0] = __builtin_amdgcn_fmed3f(l[0], x, 0x1.fffffep127f);
}

// x of another lane of the same row of 16, by a DPP lane pattern
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Eight consecutive io-typed values of a row, as floats.
template <bool F32IO>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (F32IO) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem);
    v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
    v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
  }
}

// Candidate-count buckets compiled: 1 (argmin modes), 4, 8.
// One workgroup's work: head blockIdx.y, segment block bx.
template <int D, bool F32IO, bool KEY, int KC, int R, int NW>
__device__ __forceinline__ void append_body(const AppendParams& p, int bx) {
  constexpr int NTH = 64 * NW;  // threads per workgroup
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NG = D / 16;      // residual groups (= MFMA k-steps of 16 channels)
  constexpr int ROW = D + kPad;   // LDS row pitch (bf16 elements)
  // tracked keys: K_c, the next one and spares for rescoring (two for Keys,
  // whose lists otherwise fall back to the all-centre search for about one
  // token in 3000; one for Values)
  constexpr int L = KEY ? KC + 3 : KC + 2;
  constexpr int NV = D / 8;       // 8-value chunks per row

  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const int C = p.C;
  const int Cpad = p.Cpad;

  __bf16* mu_hi = reinterpret_cast<__bf16*>(smem);
  __bf16* mu_lo = mu_hi + Cpad * ROW;  // used for fp32 activations only
  float* init = reinterpret_cast<float*>(mu_hi + Cpad * ROW * (F32IO ? 2 : 1));
  float* s_lds = init + Cpad;
  double* u_lds = reinterpret_cast<double*>(s_lds + D);  // [D][R] fp64 (Keys with PSAC only)
  // per-wave row buffer for the rare all-centre search (D words per wave)
  uint32_t* row_lds = reinterpret_cast<uint32_t*>(u_lds + D * R) + wave * D;

  const void* mu_g = F32IO ? static_cast<const void*>(static_cast<const float*>(p.mu) + (int64_t)h * C * D)
                           : static_cast<const void*>(static_cast<const uint16_t*>(p.mu) + (int64_t)h * C * D);

  // ---- stage the codebook, the accumulator start values, s and U in LDS ----
  // Start values, s and U: loaded first, unconditionally from clamped
  // indices (a conditional load would wait for itself inside its branch), so
  // that their latency overlaps the codebook's.
  constexpr int IPT = (512 + NTH - 1) / NTH;                   // start values per thread (C <= 512)
  constexpr int UPT = (D * (R > 0 ? R : 1) + NTH - 1) / NTH;  // U entries per thread
  float iv[IPT];
  double uv[UPT];
#pragma unroll
  for (int u = 0; u < IPT; ++u) {
    const int c = u * NTH + (int)threadIdx.x;
    iv[u] = p.norm_half[(int64_t)h * C + min(c, C - 1)];
  }
  const int jt = min((int)threadIdx.x, D - 1);
  float sj = p.sens[(int64_t)h * D + jt];  // the block holds s also under QWM_UNIFORM_SENS
  if constexpr (KEY && R > 0) {
#pragma unroll
    for (int u = 0; u < UPT; ++u) {
      const int e = u * NTH + (int)threadIdx.x;
      uv[u] = p.u64[(int64_t)h * D * R + min(e, D * R - 1)];
    }
  }

  // bf16 codebooks: every global load of a thread is issued before its LDS
  // stores, so staging costs about one memory latency (16 row chunks per
  // thread cover every supported C in one round)
  if constexpr (F32IO) {
    for (int e = threadIdx.x; e < Cpad * NV; e += NTH) {
      const int c = e / NV, j8 = (e % NV) * 8;
      float v[8];
      if (c < C) load8<true>(mu_g, (int64_t)c * D + j8, v);
      else for (int i = 0; i < 8; ++i) v[i] = 0.f;
      bf16x8 hi, lo;
      for (int i = 0; i < 8; ++i) {
        hi[i] = (__bf16)v[i];
        lo[i] = (__bf16)(v[i] - (float)hi[i]);
      }
      *reinterpret_cast<bf16x8*>(mu_hi + c * ROW + j8) = hi;
      *reinterpret_cast<bf16x8*>(mu_lo + c * ROW + j8) = lo;
    }
  } else {
    constexpr int CH = 16;
    const int total = Cpad * NV;
    for (int base = 0; base < total; base += CH * NTH) {
      uint4 w[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int e = min(base + u * NTH + (int)threadIdx.x, total - 1);
        const int c = e / NV, j8 = (e % NV) * 8;
        w[u] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(mu_g) + (int64_t)min(c, C - 1) * D + j8);
        if (c >= C) w[u] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int e = base + u * NTH + (int)threadIdx.x;
        if (e < total) *reinterpret_cast<uint4*>(mu_hi + (e / NV) * ROW + (e % NV) * 8) = w[u];
      }
    }
  }
  {
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int c = u * NTH + (int)threadIdx.x;
      if (c < Cpad) init[c] = c < C ? -iv[u] : -3.0e38f;
    }
    if (p.uniform) sj = 1.f;
    if ((int)threadIdx.x < D) s_lds[threadIdx.x] = sj;
    if constexpr (KEY && R > 0) {
#pragma unroll
      for (int u = 0; u < UPT; ++u) {
        const int e = u * NTH + (int)threadIdx.x;
        if (e < D * R) u_lds[e] = uv[u];
      }
    }
  }
  __syncthreads();

  // ---- segments of this wave ----
  const int seg_base = (bx * NW + wave) * kSegsPerWave;
  int seg_len[kSegsPerWave], seg_first[kSegsPerWave], seg_pos[kSegsPerWave], seg_frame[kSegsPerWave];
#pragma unroll
  for (int s = 0; s < kSegsPerWave; ++s) {
    const int g = seg_base + s;
    if (g < p.total_segs) {
      const int fr = g / p.segs_per_frame, sif = g % p.segs_per_frame;
      seg_frame[s] = fr;
      seg_pos[s] = sif * kSegTokens;
      seg_first[s] = fr * p.F + sif * kSegTokens;
      seg_len[s] = min(kSegTokens, p.F - sif * kSegTokens);
    } else {
      seg_frame[s] = 0; seg_pos[s] = 0; seg_first[s] = 0; seg_len[s] = 0;
    }
  }
  if (seg_len[0] == 0) return;  // wave-uniform; no workgroup barrier follows

  const void* xin = F32IO ? static_cast<const void*>(static_cast<const float*>(p.x) + (int64_t)h * p.head_stride)
                          : static_cast<const void*>(static_cast<const uint16_t*>(p.x) + (int64_t)h * p.head_stride);

  // ---- 1. screen ----
  // Keys screen one segment per pass (x needs hi and lo parts: fewer live
  // registers); Values screen both segments together and share each A
  // fragment between two MFMAs.  Each pass is software-pipelined: the MFMAs
  // of centre block b+1 are issued while the keys of block b are inserted.
  constexpr bool kLo = KEY || F32IO;  // x needs a bf16 lo part
  constexpr int SPP = kLo ? 1 : kSegsPerWave;  // segments per screen pass
  constexpr int RW = D / 4;  // bf16 words of one lane's half row (8 channels per k-step)
  const uint32_t pb = 32 - __builtin_clz((uint32_t)(Cpad - 1));
  const uint32_t mask = (1u << pb) - 1u;
  const int nblk = Cpad >> 5;  // even: Cpad is a multiple of 64
  // ~mask held in a VGPR, so the key is one v_and_or_b32 with the uniform index
  uint32_t keep = ~mask;
  asm volatile("" : "+v"(keep));
  float lst[kSegsPerWave][L];
  float ksq[kSegsPerWave];  // this lane's half of ||k||_s^2 (Values: ||v||^2)
  // bf16 Values keep the half rows (their MFMA operand) for the lane phase;
  // Keys, whose operand is s * k in hi + lo parts, load the row again
  constexpr bool kKeepRow = !kLo;
  uint32_t raw[kSegsPerWave][kKeepRow ? RW : 1];
#pragma unroll
  for (int pass = 0; pass < kSegsPerWave / SPP; ++pass) {
    // compiler barrier: s is read from LDS again in each pass rather than kept
    // in registers across the screen (it emits no instruction)
    asm volatile("" ::: "memory");
    bf16x8 xh[SPP][NG];
    bf16x8 xl[SPP][kLo ? NG : 1];
#pragma unroll
    for (int sp = 0; sp < SPP; ++sp) {
      const int s = pass * SPP + sp;
      const bool valid = l32 < seg_len[s];
      // rows of invalid lanes are clamped to a real token and zeroed after the load
      const int64_t row = (int64_t)(seg_first[s] + (valid ? l32 : 0)) * p.token_stride;
      float q = 0.f;
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        const int c0 = 16 * ks + 8 * half;
        float v[8];
        if constexpr (F32IO) {
          load8<true>(xin, row + c0, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = valid ? v[i] : 0.f;
        } else {
          uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xin) + row + c0);
          if (!valid) w = make_uint4(0, 0, 0, 0);
          if constexpr (kKeepRow) {
            raw[s][4 * ks + 0] = w.x;
            raw[s][4 * ks + 1] = w.y;
            raw[s][4 * ks + 2] = w.z;
            raw[s][4 * ks + 3] = w.w;
          }
          v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
          v[4] = bf_lo(w.z); v[5] = bf_hi(w.z); v[6] = bf_lo(w.w); v[7] = bf_hi(w.w);
          // bf16 Values: the loaded words are the MFMA operand (x = v exactly)
          if constexpr (!kLo) xh[sp][ks] = __builtin_bit_cast(bf16x8, w);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xf = KEY ? s_lds[c0 + i] * v[i] : v[i];
          q = fmaf(xf, v[i], q);
          if constexpr (kLo) {
            const __bf16 hb = (__bf16)xf;
            xh[sp][ks][i] = hb;
            xl[sp][ks][i] = (__bf16)(xf - (float)hb);
          }
        }
      }
      // pinned here, so the unpacked row is not kept alive to form it later
      asm volatile("" : "+v"(q));
      ksq[s] = q;
#pragma unroll
      for (int i = 0; i < L; ++i) lst[s][i] = -INFINITY;
    }

    // accumulators of centre block blk: start values, then the MFMA chain.
    // Lane (token l32, half) holds centres blk*32 + 8(i/4) + 4*half + i%4.
    auto mfma_blk = [&](int blk, f32x16 (&acc)[SPP]) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 v4 = *reinterpret_cast<const float4*>(init + blk * 32 + 8 * q4 + 4 * half);
#pragma unroll
        for (int sp = 0; sp < SPP; ++sp) {
          acc[sp][4 * q4 + 0] = v4.x;
          acc[sp][4 * q4 + 1] = v4.y;
          acc[sp][4 * q4 + 2] = v4.z;
          acc[sp][4 * q4 + 3] = v4.w;
        }
      }
      const __bf16* arow = mu_hi + (blk * 32 + l32) * ROW + 8 * half;
#pragma unroll
      for (int ks = 0; ks < NG; ++ks) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(arow + 16 * ks);
#pragma unroll
        for (int sp = 0; sp < SPP; ++sp) {
          acc[sp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xh[sp][ks], acc[sp], 0, 0, 0);
          if constexpr (kLo) acc[sp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, xl[sp][ks], acc[sp], 0, 0, 0);
        }
        if constexpr (F32IO) {
          const bf16x8 alo = *reinterpret_cast<const bf16x8*>(mu_lo + (blk * 32 + l32) * ROW + 8 * half + 16 * ks);
#pragma unroll
          for (int sp = 0; sp < SPP; ++sp)
            acc[sp] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, xh[sp][ks], acc[sp], 0, 0, 0);
        }
      }
    };
    // keys of block blk: the score with its low pb bits replaced by the centre
    // index; the lane-half bit (4 * half) is added after the screen, so the
    // index here is wave-uniform
    auto topl_blk = [&](int blk, const f32x16 (&acc)[SPP]) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint32_t c = (uint32_t)(blk * 32 + 8 * (i / 4) + (i % 4));
        asm volatile("" : "+s"(c));  // one scalar operand: the key is one v_and_or_b32
#pragma unroll
        for (int sp = 0; sp < SPP; ++sp)
          topl_insert<L>(lst[pass * SPP + sp], __uint_as_float((__float_as_uint(acc[sp][i]) & keep) | c));
      }
    };
    // issue order of one half step: the start values and first A fragment,
    // then each MFMA followed by its share of the insertions and the next
    // fragment read, so the matrix core and the VALU work side by side
    constexpr int NMF = NG * SPP * (kLo ? 2 : 1) + (F32IO ? NG * SPP : 0);  // MFMAs per block
    constexpr int NVA = 16 * SPP * (L + 1);                                  // key VALU per block
    auto interleave = [&]() {
      __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (NVA + NMF - 1) / NMF, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    };
    f32x16 acc0[SPP], acc1[SPP];
    mfma_blk(0, acc0);
    int blk = 0;
    for (; blk + 2 < nblk; blk += 2) {
      mfma_blk(blk + 1, acc1);
      topl_blk(blk, acc0);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
      mfma_blk(blk + 2, acc0);
      topl_blk(blk + 1, acc1);
      interleave();
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_blk(blk + 1, acc1);
    topl_blk(blk, acc0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    topl_blk(blk + 1, acc1);
  }

  // the lane-half bit of the centre index joins the keys (-inf entries stay)
  const uint32_t hbit = (uint32_t)half << 2;
#pragma unroll
  for (int s = 0; s < kSegsPerWave; ++s)
#pragma unroll
    for (int i = 0; i < L; ++i) {
      const float k = lst[s][i];
      lst[s][i] = k > -INFINITY ? __uint_as_float(__float_as_uint(k) | hbit) : k;
    }

  // Lane = token from here: lane t takes token t of segment 0, lane t + 32
  // token t of segment 1.  One v_permlane32_swap per register moves the upper
  // half's segment-0 data down and the lower half's segment-1 data up, so each
  // lane ends with both halves (lists, ||k||^2 parts, row words) of its token.
  auto swap32 = [](uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    a = r[0];
    b = r[1];
  };
  float mylst[L];
  {
    float other[L];
#pragma unroll
    for (int i = 0; i < L; ++i) {
      uint32_t a = __float_as_uint(lst[0][i]), b = __float_as_uint(lst[1][i]);
      swap32(a, b);
      mylst[i] = __uint_as_float(a);
      other[i] = __uint_as_float(b);
    }
#pragma unroll
    for (int i = 0; i < L; ++i) topl_insert<L>(mylst, other[i]);
  }
  float myksq;
  {
    uint32_t a = __float_as_uint(ksq[0]), b = __float_as_uint(ksq[1]);
    swap32(a, b);
    myksq = __uint_as_float(a) + __uint_as_float(b);
  }

  // ---- 2. certification ----
  // key_c is F~_c with the centre index in its low pb bits.  For every centre
  //   |key_c - F_c| <= e_c + r |key_c|,
  // e_c = (2 (n + 1) 2^-24 + 2^-17) scale_c bounds the fp32 accumulation of the
  // n products and the start value in any order at up to one ulp per operation,
  // plus the bf16 hi/lo split of x (and of mu for fp32 inputs);
  // scale_c = ||mu_c||_s^2 / 2 + ||k||_s ||mu_c||_s bounds every partial sum of
  // centre c's score (Cauchy-Schwarz), and r = 2^(pb-23) is the truncation of
  // the index bits.  The candidate set is certain when the weakest tracked
  // member's lower bar clears the upper bars of all outsiders.
  constexpr int NACC = (kLo ? 2 : 1) * D + (F32IO ? D : 0) + 1;
  const float mx = p.head_max[h * 4 + p.head_max_slot];
  const int kc = p.Kc;
  const int sidx = half;  // lane = token from here: segment `half`, token l32
  const int mylen = sidx ? seg_len[1] : seg_len[0];
  const bool valid = l32 < mylen;
  const int first = sidx ? seg_first[1] : seg_first[0];
  const int pos = (sidx ? seg_pos[1] : seg_pos[0]) + l32;  // token position inside its frame
  const int frame = p.frame0 + (sidx ? seg_frame[1] : seg_frame[0]);
  const int tok_rel = first + (valid ? l32 : 0);
  const int64_t tok = p.tok0 + tok_rel;
  // The token's row in registers: bf16 Values take the screen's half rows
  // (zero on invalid lanes); other rows are loaded again (invalid lanes hold a
  // clamped real row).  Invalid lanes are masked at every reduction and store.
  uint32_t kw[F32IO ? D : D / 2];
  if constexpr (F32IO) {
    const int64_t krow = (int64_t)tok_rel * p.token_stride;
#pragma unroll
    for (int j8 = 0; j8 < NV; ++j8) {
      float v[8];
      load8<true>(xin, krow + 8 * j8, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) kw[8 * j8 + i] = __float_as_uint(v[i]);
    }
  } else if constexpr (!kKeepRow) {
    const int64_t krow = (int64_t)tok_rel * p.token_stride;
#pragma unroll
    for (int j8 = 0; j8 < NV; ++j8) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xin) + krow + 8 * j8);
      kw[4 * j8 + 0] = w.x;
      kw[4 * j8 + 1] = w.y;
      kw[4 * j8 + 2] = w.z;
      kw[4 * j8 + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        swap32(raw[0][4 * g + i], raw[1][4 * g + i]);
        kw[8 * g + i] = raw[0][4 * g + i];      // channels 16g + 2i, 16g + 2i + 1
        kw[8 * g + 4 + i] = raw[1][4 * g + i];  // channels 16g + 8 + 2i, ...
      }
  }
  // Register fence on the packed row: an empty asm that the compiler must
  // assume rewrites the words, so unpacked copies are not kept alive across
  // phases (it emits no instruction).
  auto fence_row = [&]() {
#pragma unroll
    for (int i = 0; i < (F32IO ? D : D / 2); ++i) asm volatile("" : "+v"(kw[i]));
  };
  // Bars of every tracked entry from its own centre's norm (the nearest centres
  // are typically far from the largest norm); the untracked centres, whose keys
  // are at most the last tracked key, are bounded with the head's largest norm
  // (the upper bar is increasing in the key).
  const float ecoef = (2.f * (NACC + 1) * 0x1p-24f + 0x1p-17f) * 1.001f;
  const float xn = 1.01f * sqrtf(fmaxf(myksq, 0.f));
  const float rr = __uint_as_float((uint32_t)(127 + (int)pb - 23) << 23);
  float lo_e[L], hi_e[L];
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const float k = mylst[i];
    const int ci = min((int)(__float_as_uint(k) & mask), C - 1);
    const float nh = fmaxf(-init[ci], 0.f);  // ||mu_c||^2 / 2 (weighted for Keys)
    const float e = ecoef * (nh + xn * sqrtf(2.f * nh) * 1.0001f) + 1e-30f;
    const bool fin = k > -INFINITY;  // -inf: fewer centres than tracked entries
    lo_e[i] = fin ? k - e - rr * fabsf(k) : -INFINITY;
    hi_e[i] = fin ? k + e + rr * fabsf(k) : -INFINITY;
  }
  const float klast = mylst[L - 1];
  const float u_hi = (C <= L) ? -INFINITY : klast + ecoef * (0.5f * mx * mx + xn * mx) + 1e-30f + rr * fabsf(klast);
  float H = u_hi, Lmin = INFINITY;  // best outsider's upper bar, weakest member's lower bar
#pragma unroll
  for (int i = 0; i < L; ++i) {
    if (i >= kc) H = fmaxf(H, hi_e[i]);
    else Lmin = fminf(Lmin, lo_e[i]);
  }
  const bool certain = (C <= kc) || (Lmin > H);
  const bool list_covers = u_hi < Lmin;

  // ---- 3. lane = token ----
  // The token's channels are re-read per residual group from memory (the row
  // was just streamed in, so these reads hit the caches); the group loops stay
  // rolled, which keeps the live state to one group at a time.
  // The 16 channels of residual group g (g is wave-uniform): a switch on g
  // becomes scalar branches, so the row stays in registers with static indices.
  auto load_k16 = [&](int g, float (&k)[16]) {
    constexpr int WPG = F32IO ? 16 : 8;  // row words per group
    uint32_t w[WPG];
    switch (g) {
#define QWM_GROUP_CASE(G)                                              \
      case G:                                                          \
        if constexpr (G < NG) {                                        \
          _Pragma("unroll") for (int i = 0; i < WPG; ++i) w[i] = kw[G * WPG + i]; \
        }                                                              \
        break;
      QWM_GROUP_CASE(0) QWM_GROUP_CASE(1) QWM_GROUP_CASE(2) QWM_GROUP_CASE(3)
      QWM_GROUP_CASE(4) QWM_GROUP_CASE(5) QWM_GROUP_CASE(6) QWM_GROUP_CASE(7)
#undef QWM_GROUP_CASE
      default:
        break;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (F32IO) k[i] = __uint_as_float(w[i]);
      else k[i] = (i & 1) ? bf_hi(w[i >> 1]) : bf_lo(w[i >> 1]);
    }
  };
  auto mu_row16 = [&](int c, int g, float (&m)[16]) {
    float a[8], b[8];
    if constexpr (F32IO) {
      load8<true>(mu_g, (int64_t)c * D + 16 * g, a);
      load8<true>(mu_g, (int64_t)c * D + 16 * g + 8, b);
    } else {
      const uint4* q = reinterpret_cast<const uint4*>(mu_hi + c * ROW + 16 * g);
      uint4 w0 = q[0], w1 = q[1];
      a[0] = bf_lo(w0.x); a[1] = bf_hi(w0.x); a[2] = bf_lo(w0.y); a[3] = bf_hi(w0.y);
      a[4] = bf_lo(w0.z); a[5] = bf_hi(w0.z); a[6] = bf_lo(w0.w); a[7] = bf_hi(w0.w);
      b[0] = bf_lo(w1.x); b[1] = bf_hi(w1.x); b[2] = bf_lo(w1.y); b[3] = bf_hi(w1.y);
      b[4] = bf_lo(w1.z); b[5] = bf_hi(w1.z); b[6] = bf_lo(w1.w); b[7] = bf_hi(w1.w);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) { m[i] = a[i]; m[8 + i] = b[i]; }
  };

  int cand[KC];
  // tie-break value for QSAC stage 2 (smaller is better), on the -F scale:
  // -key with its index bits cleared (so that equal scores tie and the lower
  // index wins, not the larger index field), or (D - ||k||_s^2) / 2 for
  // centres that were rescored exactly
  auto key_tie = [&](float key) { return -__uint_as_float(__float_as_uint(key) & ~mask); };
  float tieD[KC];
#pragma unroll
  for (int i = 0; i < KC; ++i) {
    // clamp: only non-finite inputs can produce an index outside [0, C)
    cand[i] = min((int)(__float_as_uint(mylst[i]) & mask), C - 1);
    tieD[i] = key_tie(mylst[i]);
  }

  // D_c = sum_j s_j (k_j - mu_cj)^2 in fp64 for one centre, the row given by
  // `row_word` (register row, or a broadcast one).  For bf16 inputs k - mu is
  // exact in fp32; the products and the sum are fp64.
  auto exact_d_row = [&](int c, auto&& row_words) -> double {
    double dd = 0.0;
#pragma unroll 1
    for (int g = 0; g < NG; ++g) {
      float k[16], m[16];
      row_words(g, k);
      mu_row16(c, g, m);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const double df = F32IO ? (double)k[i] - (double)m[i] : (double)(k[i] - m[i]);
        dd = fma((double)s_lds[16 * g + i] * df, df, dd);
      }
    }
    return dd;
  };
  // exact top-K_c buffer, ascending (D, c)
  double bd[KC];
  int bc[KC];
  auto reset_best = [&]() {
#pragma unroll
    for (int i = 0; i < KC; ++i) { bd[i] = INFINITY; bc[i] = 0x7fffffff; }
  };
  auto insert = [&](double dd, int c) {
#pragma unroll
    for (int i = KC - 1; i >= 0; --i) {
      const int ip = i > 0 ? i - 1 : 0;
      const bool before_prev = i > 0 && (dd < bd[ip] || (dd == bd[ip] && c < bc[ip]));
      const bool before_this = dd < bd[i] || (dd == bd[i] && c < bc[i]);
      if (before_prev) { bd[i] = bd[i - 1]; bc[i] = bc[i - 1]; }
      else if (before_this) { bd[i] = dd; bc[i] = c; }
    }
  };

  // (1) Band rescoring.  A tracked member (i < K_c) whose lower bar clears every
  // outsider's upper bar is surely a candidate; a tracked entry whose upper bar
  // is below every member's lower bar surely is not.  The rest (the band) is
  // rescored exactly and fills the slots the sure members leave.
  const bool need_band = !certain && list_covers && valid;
  uint32_t sure_bits = 0, band_bits = 0;
#pragma unroll
  for (int i = 0; i < L; ++i) {
    const bool sure = i < kc && lo_e[i] > H;
    const bool out = i >= kc && hi_e[i] < Lmin;
    if (sure) sure_bits |= 1u << i;
    if (!sure && !out && mylst[i] > -INFINITY) band_bits |= 1u << i;
  }
  if (__any(need_band)) {
    if (p.counters && lane == 0) atomicAdd(p.counters + (KEY ? 0 : 2), (uint32_t)__popcll(__ballot(need_band)));
    reset_best();
    // Requests (lane t, tracked entry i) are served four at a time by the
    // whole wave: request q takes lanes 16q..16q+15, each summing CPL channels
    // of D_c in fp64, then a 16-lane reduction; the owner lane inserts the
    // result.  The request lists are wave-uniform (scalar), so only the
    // requests themselves cost work, not every lane of a wave that has one.
    constexpr int CPL = D / 16;  // channels per lane of a request
    const int q = lane >> 4, part = lane & 15;
    const uint32_t tok_bits = (uint32_t)tok_rel;
#pragma unroll 1
    for (int i = 0; i < L; ++i) {
      uint64_t req = __ballot(need_band && ((band_bits >> i) & 1u));
      if (req == 0) continue;
      float key_i = mylst[0];
#pragma unroll
      for (int e = 1; e < L; ++e)
        if (e == i) key_i = mylst[e];
      const uint32_t c_bits = __float_as_uint(key_i) & mask;
      while (req) {
        int tq[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          tq[r] = req ? __builtin_ctzll(req) : -1;
          req &= req ? req - 1 : 0ull;
        }
        // this lane's request: owner lane, centre and token row (uniform reads)
        int my_t = -1, my_c = 0, my_tok = 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tq[r];
          const int cr = t >= 0 ? (int)__builtin_amdgcn_readlane(c_bits, t) : 0;
          const int kr = t >= 0 ? (int)__builtin_amdgcn_readlane(tok_bits, t) : 0;
          if (q == r) { my_t = t; my_c = cr; my_tok = kr; }
        }
        double part_d = 0.0;
        if (my_t >= 0 && my_c < C) {
          const int64_t row = (int64_t)my_tok * p.token_stride + CPL * part;
          float kv[CPL], mv[CPL];
          if constexpr (F32IO) {
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              kv[j] = static_cast<const float*>(xin)[row + j];
              mv[j] = static_cast<const float*>(mu_g)[(int64_t)my_c * D + CPL * part + j];
            }
          } else {
            const uint16_t* kp = static_cast<const uint16_t*>(xin) + row;
            const uint16_t* mp = reinterpret_cast<const uint16_t*>(mu_hi) + my_c * ROW + CPL * part;
#pragma unroll
            for (int j = 0; j < CPL; j += 2) {
              const uint32_t kw2 = *reinterpret_cast<const uint32_t*>(kp + j);
              const uint32_t mw2 = *reinterpret_cast<const uint32_t*>(mp + j);
              kv[j] = bf_lo(kw2); kv[j + 1] = bf_hi(kw2);
              mv[j] = bf_lo(mw2); mv[j + 1] = bf_hi(mw2);
            }
          }
#pragma unroll
          for (int j = 0; j < CPL; ++j) {
            const double df = F32IO ? (double)kv[j] - (double)mv[j] : (double)(kv[j] - mv[j]);
            part_d = fma((double)s_lds[CPL * part + j] * df, df, part_d);
          }
        }
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) part_d += __shfl_xor(part_d, off);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = tq[r];
          if (t < 0) break;
          const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)__double_as_longlong(part_d), 16 * r);
          const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)__double_as_longlong(part_d) >> 32), 16 * r);
          const double dq = __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
          const int cq = (int)(__float_as_uint(key_i) & mask);
          if (lane == t && cq < C) insert(dq, cq);
        }
      }
    }
    if (need_band) {
      // sure members first (in list order), then the exact winners in order
      int n_sure = 0;
#pragma unroll
      for (int i = 0; i < L; ++i) {
        if ((sure_bits >> i) & 1u) {
          const int c = min((int)(__float_as_uint(mylst[i]) & mask), C - 1);
#pragma unroll
          for (int q = 0; q < KC; ++q)
            if (q == n_sure) { cand[q] = c; tieD[q] = key_tie(mylst[i]); }
          ++n_sure;
        }
      }
#pragma unroll
      for (int q = 0; q < KC; ++q) {
        const int src = q - n_sure;  // rank among the rescored entries
        if (q >= n_sure && q < kc) {
          int c = bc[0];
          double dd = bd[0];
#pragma unroll
          for (int r = 1; r < KC; ++r)
            if (r == src) { c = bc[r]; dd = bd[r]; }
          cand[q] = min(c, C - 1);
          tieD[q] = (float)(0.5 * (dd - (double)myksq));
        }
      }
    }
  }

  // (2) Rare: the tracked list does not hold every possible candidate.  The
  // whole wave searches all centres for one such token at a time: its row is
  // broadcast to scalar registers and lane l scores centres l, l+64, ...
  uint64_t full = __ballot(!certain && !list_covers && valid);
  if (p.counters && full && lane == 0) atomicAdd(p.counters + (KEY ? 1 : 3), (uint32_t)__popcll(full));
  while (full) {
    const int t = __builtin_ctzll(full);
    full &= full - 1;
    constexpr int KWN = F32IO ? D : D / 2;
    if (lane == t) {
#pragma unroll
      for (int i = 0; i < KWN; i += 4)
        *reinterpret_cast<uint4*>(row_lds + i) = make_uint4(kw[i], kw[i + 1], kw[i + 2], kw[i + 3]);
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the row is in LDS for every lane
    auto bcast_k16 = [&](int g, float (&k)[16]) {
      constexpr int WPG = F32IO ? 16 : 8;
      const uint32_t* src = row_lds + g * WPG;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (F32IO) k[i] = __uint_as_float(src[i]);
        else k[i] = (i & 1) ? bf_hi(src[i >> 1]) : bf_lo(src[i >> 1]);
      }
    };
    reset_best();
#pragma unroll 1
    for (int c = lane; c < C; c += 64) insert(exact_d_row(c, bcast_k16), c);
    // K_c rounds of a wave-wide lexicographic (D, c) minimum
    const float ksq_t = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(myksq), t));
#pragma unroll
    for (int q = 0; q < KC; ++q) {
      double wd = bd[0];
      int wc = bc[0];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double od = __shfl_xor(wd, off);
        const int oc = __shfl_xor(wc, off);
        if (od < wd || (od == wd && oc < wc)) { wd = od; wc = oc; }
      }
      if (bc[0] == wc) {  // the owner pops its head
#pragma unroll
        for (int r = 0; r < KC - 1; ++r) { bd[r] = bd[r + 1]; bc[r] = bc[r + 1]; }
        bd[KC - 1] = INFINITY;
        bc[KC - 1] = 0x7fffffff;
      }
      if (lane == t && q < kc) {
        cand[q] = min(wc, C - 1);
        tieD[q] = (float)(0.5 * (wd - (double)ksq_t));
      }
    }
    __builtin_amdgcn_wave_barrier();  // all reads of this row precede the next write
  }

  // ---- QSAC stage 2: expected INT2 logit perturbation of each candidate ----
  fence_row();
  int chosen = cand[0];
  if constexpr (KEY && KC > 1) {
    if (p.use_range) {
      double P[KC];
#pragma unroll
      for (int i = 0; i < KC; ++i) P[i] = 0.0;
      if (p.s2mode == 0) {
        // P_c = sum_g S_g range_g(k - mu_c)^2 for every tracked candidate at once:
        // each residual group of the row is unpacked once for all K_c centres
        const double* sg = p.sgroup + (int64_t)h * NG;
#pragma unroll 1
        for (int g = 0; g < NG; ++g) {
          float k[16];
          load_k16(g, k);
          const double sgv = p.uniform ? 16.0 : sg[g];
#pragma unroll
          for (int i = 0; i < KC; ++i) {
            float m[16];
            mu_row16(cand[i], g, m);
            float lo = k[0] - m[0], hi = lo;
#pragma unroll
            for (int j = 1; j < 16; ++j) {
              const float rho = k[j] - m[j];
              lo = fminf(lo, rho);
              hi = fmaxf(hi, rho);
            }
            const double rg = (double)hi - (double)lo;
            P[i] = fma(sgv, rg * rg, P[i]);
          }
        }
      } else {
        // ablation scores on the candidate's actual INT2 error: group g of the
        // token's residual against centre c, quantized with the group's own
        // (zero, scale) by the tile arithmetic below; e = rho - rho_hat (exact
        // in fp64)
        auto err16 = [&](int c, int g, double (&e)[16]) {
          float k[16], m[16], rho[16];
          load_k16(g, k);
          mu_row16(c, g, m);
          rho[0] = k[0] - m[0];
          float lo = rho[0], hi = rho[0];
#pragma unroll
          for (int j = 1; j < 16; ++j) {
            rho[j] = k[j] - m[j];
            lo = fminf(lo, rho[j]);
            hi = fmaxf(hi, rho[j]);
          }
          const float zf = half_bits_to_float(to_half_bits(lo));
          const float sf = half_bits_to_float(to_half_bits((hi - lo) / 3.0f));
          const bool zs = sf == 0.f;
          const float t1 = zs ? INFINITY : zf + 0.5f * sf;
          const float t2 = zs ? INFINITY : zf + 1.5f * sf;
          const float t3 = zs ? INFINITY : zf + 2.5f * sf;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float code = (float)((int)(rho[j] >= t1) + (int)(rho[j] >= t2) + (int)(rho[j] >= t3));
            e[j] = (double)rho[j] - (double)fmaf(code, sf, zf);
          }
        };
        // one candidate at a time (a uniform loop: the error rows stay in
        // registers with static indices).  s2mode 1, the diagonal form:
        // P_c = sum_j s_j e_j^2.  s2mode 2, the full form: P_c = e^T M e =
        // sum_g [e_g^T M_gg e_g + 2 sum_{g' < g} e_g^T M_gg' e_g'], block by
        // block with both groups' errors recomputed (M is symmetric and read
        // wave-uniformly).
        const double* M = p.moment + (int64_t)h * D * D;
        const bool full = p.s2mode == 2;
#pragma unroll 1
        for (int ci = 0; ci < KC; ++ci) {
          int c = cand[0];
#pragma unroll
          for (int i = 1; i < KC; ++i) c = ci == i ? cand[i] : c;
          double acc = 0.0;
#pragma unroll 1
          for (int g = 0; g < NG; ++g) {
            double eg[16];
            err16(c, g, eg);
            if (!full) {
#pragma unroll
              for (int j = 0; j < 16; ++j) acc = fma((double)s_lds[16 * g + j] * eg[j], eg[j], acc);
              continue;
            }
#pragma unroll 1
            for (int gp = 0; gp <= g; ++gp) {
              double ep[16];
              if (gp == g) {
#pragma unroll
                for (int j = 0; j < 16; ++j) ep[j] = eg[j];
              } else {
                err16(c, gp, ep);
              }
              const double* mb = M + (int64_t)(16 * g) * D + 16 * gp;
              double blk = 0.0;
#pragma unroll
              for (int a = 0; a < 16; ++a) {
                double t = 0.0;
#pragma unroll
                for (int b = 0; b < 16; ++b) t = fma(mb[a * D + b], ep[b], t);
                blk = fma(eg[a], t, blk);
              }
              acc = fma(gp == g ? 1.0 : 2.0, blk, acc);
            }
          }
#pragma unroll
          for (int i = 0; i < KC; ++i) P[i] = ci == i ? acc : P[i];
        }
      }
      double bestP = INFINITY;
      float bestD = INFINITY;
      int best = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < KC; ++i) {
        const int c = cand[i];
        const bool better = (P[i] < bestP) || (P[i] == bestP && (tieD[i] < bestD || (tieD[i] == bestD && c < best)));
        if (i < kc && c < C && better) { bestP = P[i]; bestD = tieD[i]; best = c; }
      }
      chosen = best < C ? best : cand[0];  // all-NaN scores keep a valid index
    }
  }

  // ---- INT2 residual tiles and PSAC ----
  fence_row();
  const int T = p.T;
  const int tile = frame * p.tpf + pos / T;
  const int64_t slot = (int64_t)h * p.Ncap + tok;
  // PSAC accumulates c = U^T e in passes of at most 16 columns (two passes at
  // R = 32: the second recomputes the residual codes and stores nothing, so
  // that the fp64 accumulators and U rows of one pass fit in registers)
  constexpr int RC = R > 16 ? 16 : (R > 0 ? R : 1);  // columns per pass
  constexpr int NPASS = R > 16 ? 2 : 1;
  float c32[R > 0 ? R : 1];
  const double* U = u_lds;

#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    double cacc[RC];
#pragma unroll
    for (int i = 0; i < RC; ++i) cacc[i] = 0.0;
#pragma unroll 1
    for (int g = 0; g < NG; ++g) {
      float k[16], m[16];
      load_k16(g, k);
      mu_row16(chosen, g, m);
      float rho[16];
      rho[0] = k[0] - m[0];
      float lo = rho[0], hi = rho[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) {
        rho[j] = k[j] - m[j];
        lo = fminf(lo, rho[j]);
        hi = fmaxf(hi, rho[j]);
      }
      if (!valid) { lo = INFINITY; hi = -INFINITY; }
      // min / max over the T lanes of the tile (T | 32, tiles lane-aligned)
      if (T > 1) { lo = fminf(lo, dpp_f<0xB1>(lo)); hi = fmaxf(hi, dpp_f<0xB1>(hi)); }    // lane ^ 1
      if (T > 2) { lo = fminf(lo, dpp_f<0x4E>(lo)); hi = fmaxf(hi, dpp_f<0x4E>(hi)); }    // lane ^ 2
      if (T > 4) { lo = fminf(lo, dpp_f<0x141>(lo)); hi = fmaxf(hi, dpp_f<0x141>(hi)); }  // 7 - lane in 8
      if (T > 8) { lo = fminf(lo, dpp_f<0x140>(lo)); hi = fmaxf(hi, dpp_f<0x140>(hi)); }  // 15 - lane in 16
      if (T > 16) { lo = fminf(lo, __shfl_xor(lo, 16)); hi = fmaxf(hi, __shfl_xor(hi, 16)); }
      const uint16_t zb = to_half_bits(lo);
      const uint16_t sb = to_half_bits((hi - lo) / 3.0f);
      const float zf = half_bits_to_float(zb);
      const float sf = half_bits_to_float(sb);
      // a zero scale codes everything as 0 (every finite residual is below +inf)
      const bool zs = sf == 0.f;
      const float t1 = zs ? INFINITY : zf + 0.5f * sf;
      const float t2 = zs ? INFINITY : zf + 1.5f * sf;
      const float t3 = zs ? INFINITY : zf + 2.5f * sf;
      uint32_t w = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t code = (uint32_t)(rho[j] >= t1) + (uint32_t)(rho[j] >= t2) + (uint32_t)(rho[j] >= t3);
        w |= code << (2 * j);
      }
      if constexpr (KEY && R > 0) {
        // c += U^T e over the group's 16 channels (this pass's columns), with
        // the next U row read while this row's FMAs run: the empty asm
        // statements (no instruction) keep the rows in order, so at most two
        // rows are live
        const double* ug = U + 16 * g * R + 16 * pass;
        double ucur[RC], unxt[RC];
#pragma unroll
        for (int i = 0; i < RC; ++i) ucur[i] = ug[i];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j + 1 < 16) {
#pragma unroll
            for (int i = 0; i < RC; ++i) unxt[i] = ug[(j + 1) * R + i];
          }
          const float rhat = fmaf((float)((w >> (2 * j)) & 3u), sf, zf);
          const double e = ((double)k[j] - (double)m[j]) - (double)rhat;
#pragma unroll
          for (int i = 0; i < RC; ++i) cacc[i] = fma(ucur[i], e, cacc[i]);
#pragma unroll
          for (int i = 0; i < RC; ++i) {
            asm volatile("" : "+v"(cacc[i]));
            ucur[i] = unxt[i];
          }
          asm volatile("" ::: "memory");
        }
      }
      if (pass == 0 && valid) {
        p.codes[slot * NG + g] = w;
        if ((pos % T) == 0) p.params[((int64_t)h * p.Pcap + tile) * NG + g] = (uint32_t)zb | ((uint32_t)sb << 16);
      }
    }
    if constexpr (KEY && R > 0) {
#pragma unroll
      for (int i = 0; i < RC; ++i) c32[RC * pass + i] = (float)cacc[i];
    }
  }

  if (!valid) return;
  if (p.idx_bytes == 1) static_cast<uint8_t*>(p.idx)[slot] = (uint8_t)chosen;
  else static_cast<uint16_t*>(p.idx)[slot] = (uint16_t)chosen;

  if constexpr (KEY && R > 0) {
    const int r = p.r;
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < R; ++i)
      if (i < r) a = fmaxf(a, fabsf(c32[i]));
    const uint16_t sgb = to_half_bits(a / 127.0f);
    const float sg = half_bits_to_float(sgb);
    int8_t n[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float v = 0.f;
      if (sg != 0.f) v = fminf(127.f, fmaxf(-127.f, rintf(c32[i] / sg)));
      n[i] = (int8_t)(int)v;
    }
    int8_t* dst = p.coef + slot * r;
    if (r == R) {
      if constexpr (R == 8) {
        uint2 pk;
        pk.x = (uint32_t)(uint8_t)n[0] | ((uint32_t)(uint8_t)n[1] << 8) | ((uint32_t)(uint8_t)n[2] << 16) | ((uint32_t)(uint8_t)n[3] << 24);
        pk.y = (uint32_t)(uint8_t)n[4] | ((uint32_t)(uint8_t)n[5] << 8) | ((uint32_t)(uint8_t)n[6] << 16) | ((uint32_t)(uint8_t)n[7] << 24);
        *reinterpret_cast<uint2*>(dst) = pk;
      } else if constexpr (R % 16 == 0) {
        // whole rows of 16-byte words (the row of token t starts at 16 R t / 16)
#pragma unroll
        for (int q = 0; q < R / 16; ++q) {
          uint32_t wv[4];
#pragma unroll
          for (int b = 0; b < 4; ++b)
            wv[b] = (uint32_t)(uint8_t)n[16 * q + 4 * b] | ((uint32_t)(uint8_t)n[16 * q + 4 * b + 1] << 8) |
                    ((uint32_t)(uint8_t)n[16 * q + 4 * b + 2] << 16) | ((uint32_t)(uint8_t)n[16 * q + 4 * b + 3] << 24);
          reinterpret_cast<uint4*>(dst)[q] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < R; ++i) dst[i] = n[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < R; ++i)
        if (i < r) dst[i] = n[i];
    }
    p.coef_scale[slot] = sgb;
  }
}

// Workgroups of 4 waves (two per CU when the codebook leaves room), or of 8
// waves for large codebooks (one workgroup per CU): 8 waves per CU either way.
template <int D, bool F32IO, bool KEY, int KC, int R, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void append_kernel(AppendParams p) {
  append_body<D, F32IO, KEY, KC, R, NW>(p, blockIdx.x);
}

// Keys (blockIdx.z == 0) and Values (blockIdx.z == 1) of the same frames in
// one launch: twice the workgroups in flight for small appends.
template <int D, bool F32IO, int KC, int R, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void append_kv_kernel(AppendParams pk, AppendParams pv) {
  if (blockIdx.z == 0) append_body<D, F32IO, true, KC, R, NW>(pk, blockIdx.x);
  else append_body<D, F32IO, false, 1, 0, NW>(pv, blockIdx.x);
}

// 8 waves when a 4-wave workgroup's LDS would not leave room for a second one
inline int waves_for(int Cpad, int D, bool f32io, int ucols) {
  return append_lds_bytes(Cpad, D, f32io, ucols, 4) > 80 * 1024 ? 8 : 4;
}

template <int D, bool F32IO, int KC, int R, int NW>
hipError_t launch_kv_nw(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream) {
  const size_t lds = std::max(append_lds_bytes(pk.Cpad, D, F32IO, R, NW), append_lds_bytes(pv.Cpad, D, F32IO, 0, NW));
  auto fn = append_kv_kernel<D, F32IO, KC, R, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int per_block = NW * kSegsPerWave;
  dim3 grid((pk.total_segs + per_block - 1) / per_block, heads, 2);
  hipLaunchKernelGGL(fn, grid, dim3(64 * NW), lds, stream, pk, pv);
  return hipGetLastError();
}

template <int D, bool F32IO, int KC, int R>
hipError_t launch_kv(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream) {
  const int nw = std::max(waves_for(pk.Cpad, D, F32IO, R), waves_for(pv.Cpad, D, F32IO, 0));
  return nw == 8 ? launch_kv_nw<D, F32IO, KC, R, 8>(pk, pv, heads, stream)
                 : launch_kv_nw<D, F32IO, KC, R, 4>(pk, pv, heads, stream);
}

template <int D, bool F32IO>
inline hipError_t dispatch_kv_d(const AppendParams& pk, const AppendParams& pv, int heads, hipStream_t stream) {
  const bool argmin = !pk.use_range || pk.Kc <= 1;
  const int rb = pk.rp;
  if (argmin) {
    if (rb == 0) return launch_kv<D, F32IO, 1, 0>(pk, pv, heads, stream);
    if (rb == 8) return launch_kv<D, F32IO, 1, 8>(pk, pv, heads, stream);
    if (rb == 16) return launch_kv<D, F32IO, 1, 16>(pk, pv, heads, stream);
    return launch_kv<D, F32IO, 1, 32>(pk, pv, heads, stream);
  }
  if (pk.Kc <= 4) {
    if (rb == 0) return launch_kv<D, F32IO, 4, 0>(pk, pv, heads, stream);
    if (rb == 8) return launch_kv<D, F32IO, 4, 8>(pk, pv, heads, stream);
    if (rb == 16) return launch_kv<D, F32IO, 4, 16>(pk, pv, heads, stream);
    return launch_kv<D, F32IO, 4, 32>(pk, pv, heads, stream);
  }
  if (rb == 0) return launch_kv<D, F32IO, 8, 0>(pk, pv, heads, stream);
  if (rb == 8) return launch_kv<D, F32IO, 8, 8>(pk, pv, heads, stream);
  if (rb == 16) return launch_kv<D, F32IO, 8, 16>(pk, pv, heads, stream);
  return launch_kv<D, F32IO, 8, 32>(pk, pv, heads, stream);
}

template <int D, bool F32IO, bool KEY, int KC, int R, int NW>
hipError_t launch_one_nw(const AppendParams& p, int heads, hipStream_t stream) {
  const size_t lds = append_lds_bytes(p.Cpad, D, F32IO, R, NW);
  auto fn = append_kernel<D, F32IO, KEY, KC, R, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int per_block = NW * kSegsPerWave;
  dim3 grid((p.total_segs + per_block - 1) / per_block, heads);
  hipLaunchKernelGGL(fn, grid, dim3(64 * NW), lds, stream, p);
  return hipGetLastError();
}

template <int D, bool F32IO, bool KEY, int KC, int R>
hipError_t launch_one(const AppendParams& p, int heads, hipStream_t stream) {
  return waves_for(p.Cpad, D, F32IO, R) == 8 ? launch_one_nw<D, F32IO, KEY, KC, R, 8>(p, heads, stream)
                                              : launch_one_nw<D, F32IO, KEY, KC, R, 4>(p, heads, stream);
}

template <int D, bool F32IO>
inline hipError_t dispatch_d(const AppendParams& p, int heads, bool key, hipStream_t stream) {
  if (!key) return launch_one<D, F32IO, false, 1, 0>(p, heads, stream);
  const bool argmin = !p.use_range || p.Kc <= 1;
  const int rb = p.rp;
  if (argmin) {
    if (rb == 0) return launch_one<D, F32IO, true, 1, 0>(p, heads, stream);
    if (rb == 8) return launch_one<D, F32IO, true, 1, 8>(p, heads, stream);
    if (rb == 16) return launch_one<D, F32IO, true, 1, 16>(p, heads, stream);
    return launch_one<D, F32IO, true, 1, 32>(p, heads, stream);
  }
  if (p.Kc <= 4) {
    if (rb == 0) return launch_one<D, F32IO, true, 4, 0>(p, heads, stream);
    if (rb == 8) return launch_one<D, F32IO, true, 4, 8>(p, heads, stream);
    if (rb == 16) return launch_one<D, F32IO, true, 4, 16>(p, heads, stream);
    return launch_one<D, F32IO, true, 4, 32>(p, heads, stream);
  }
  if (rb == 0) return launch_one<D, F32IO, true, 8, 0>(p, heads, stream);
  if (rb == 8) return launch_one<D, F32IO, true, 8, 8>(p, heads, stream);
  if (rb == 16) return launch_one<D, F32IO, true, 8, 16>(p, heads, stream);
  return launch_one<D, F32IO, true, 8, 32>(p, heads, stream);
}

}  // namespace append_detail
}  // namespace qwm

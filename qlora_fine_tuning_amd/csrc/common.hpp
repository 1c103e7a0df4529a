// Device helpers shared by the gfx950 kernels of the LoRA / QLoRA layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Tiles and launch shape of the MFMA kernels: 256 threads = 4 waves of 64 lanes, one
// 256 x 256 output tile per workgroup, contraction staged through LDS 64 at a time.
constexpr int kThreads = 256;
constexpr int kTile = 256;
constexpr int kStep = 64;

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l holds, for both operands,
// row (l & 15) of its 16-row operand and the 8 contraction indices 8*(l >> 4) .. +7;
// it receives D rows 4*(l >> 4) .. +3 of column (l & 15).
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// acc += a * b with the accumulator tied in place to AGPRs.  Written as inline asm because
// the compiler otherwise rotates loop-carried accumulators through temporary registers
// (hundreds of v_accvgpr_mov per K step).  The compiler does not see the MFMA's hazards, so:
//  * a and b must be results of LDS or memory loads (s_waitcnt-protected), never fresh VALU
//    results;
//  * mfma_acc_ready() must separate the accumulators' initialisation from the first use,
//    and mfma_drain() the last use from any other instruction that reads them.
__device__ __forceinline__ void mfma16_acc(f32x4& acc, const u32x4& a, const u32x4& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
template <int N>
__device__ __forceinline__ void mfma_acc_ready(f32x4 (&acc)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(acc[i]));
  asm volatile("s_nop 7");
}
template <int N>
__device__ __forceinline__ void mfma_drain(f32x4 (&acc)[N]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7");  // > the longest MFMA write-to-read latency
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(acc[i]));
}

// Tag for a K-loop phase that issues no copies.
struct NoCopy {
  __device__ void operator()(int) const {}
};

// A K-loop phase hook called after every MFMA (with s = 8 * row + column) instead of after
// MFMAs 1 and 5 of each row: for VALU work, which holds up the next MFMA issue when it comes
// in one block (each VALU operation takes an issue slot the MFMA stream needs), and costs far
// less in two or three operations per MFMA.
// The hook's working values (type S) live in the phase's row loop, f(s, state).
template <class S, class F>
struct EveryMfma {
  using State = S;
  F f;
};
template <class S, class F>
__device__ EveryMfma<S, F> every_mfma(F f) { return EveryMfma<S, F>{f}; }
template <class T>
struct IsEveryMfma : std::false_type {};
template <class S, class F>
struct IsEveryMfma<EveryMfma<S, F>> : std::true_type {};

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 v as hi + lo with both parts bf16 (|v - hi - lo| <= 2^-16 |v|): lets an fp32 panel
// enter a bf16 MFMA without losing the accuracy of the fp32 accumulator.
__device__ __forceinline__ void split_bf16(float v, float& hi, float& lo) {
  const uint32_t h = pack_bf16(v, 0.f) & 0xffffu;
  hi = __uint_as_float(h << 16);
  lo = v - hi;  // exact
}

// LDS operand tiles are rows of 64 bf16 (eight 16-byte chunks).  Chunk c of row r sits at
// chunk slot c ^ swz(r).
//  * swzf ("fixed"): slot c ^ (r & 7).  A fragment read (16 consecutive rows at one chunk
//    column, the four 16-lane groups at four columns) measures free of bank conflicts on
//    gfx950, and the slot depends only on the row's low 3 bits, so fragment rows 16 apart
//    differ by a constant address and all fragment reads of a wave share one register.
//  * swz: slot c ^ ((r ^ (r >> 3)) & 7), for tiles written through registers where 8 rows
//    spaced 8 apart are stored at one chunk column (the in-register transposes).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return (r << 6) + ((c ^ swz(r)) << 3); }
__device__ __forceinline__ int swzf(int r) { return r & 7; }
__device__ __forceinline__ int lds_offf(int r, int c) { return (r << 6) + ((c ^ swzf(r)) << 3); }

// ---- buffer loads ----------------------------------------------------------------------
// A buffer resource covers `bytes` bytes from `base`; loads whose offset falls outside read
// zero.  buffer_load ... lds (16 bytes per lane) writes a wave's 64 x 16 bytes to LDS at
// consecutive addresses starting at the given LDS pointer, with no VGPRs in between.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#define LORA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LORA_LDS(lds), 16, (int)voff, (int)soff, 0, 0);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
// s_waitcnt immediate for lgkmcnt(0) alone (vmcnt 63 and expcnt 7: not waited for)
constexpr int kLgkm0 = 0xC07F;
// s_waitcnt vmcnt(0): this wave's outstanding vector-memory loads (LDS DMA included) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// ds_read_b64_tr_b16: each group of 16 lanes reads a 4 x 16 block of 16-bit elements, lane
// 4i + b passing the address of elements 4b .. 4b+3 of the block's row i; lane l of the group
// receives column l of the block (rows 0..3 in order).  Two such reads give an MFMA operand
// whose 8 contraction indices run down a column of a row-major LDS tile.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 ld_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x4 join(u32x2 a, u32x2 b) { return (u32x4){a[0], a[1], b[0], b[1]}; }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x4 zero4() { return (u32x4){0u, 0u, 0u, 0u}; }
__device__ __forceinline__ f32x4 fzero4() { return (f32x4){0.f, 0.f, 0.f, 0.f}; }

// Transpose an 8x8 block of bf16 held as 8 rows of 8 (row i in in[i]) into 8 columns
// (column j in out[j]), using byte permutes.
__device__ __forceinline__ void transpose8x8(const u32x4 in[8], u32x4 out[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {      // source dword e holds columns 2e (low) and 2e+1 (high)
#pragma unroll
    for (int d = 0; d < 4; ++d) {    // destination dword d holds rows 2d (low) and 2d+1 (high)
      const uint32_t lo_src = in[2 * d][e], hi_src = in[2 * d + 1][e];
      out[2 * e][d] = __builtin_amdgcn_perm(hi_src, lo_src, 0x05040100u);
      out[2 * e + 1][d] = __builtin_amdgcn_perm(hi_src, lo_src, 0x07060302u);
    }
  }
}

// ---- int4 unpack ------------------------------------------------------------------------
// A packed dword holds 8 codes, code i (k offset i) in bits 4i .. 4i+3 as 4-bit two's
// complement.  XOR with 0x8 per nibble turns code q into the unsigned u = q + 8.  Code u is
// placed in an fp16 mantissa next to the exponent of 1024, giving the exact fp16 value
// 1024 + u (or 1024 + 16 u for a code in bits 4..7 of its byte), and one v_fma_mix_f32 widens
// it and computes
//   (1024 + u) s - 1032 s = (u - 8) s   or   (1024 + 16 u) (s / 16) - 72 s = (u - 8) s,
// exact: every product and addend fits fp32 exactly (s has at most 11 significant bits), so
// the fma returns q s itself, and one RNE pack per pair gives bf16_rne(q s): dequant8_mix.
// 17 VALU operations per 8 codes.
struct I4Mix {
  float s, s16, c0, c1;  // s, s / 16, -1032 s, -72 s
};
__device__ __forceinline__ I4Mix i4mix(float s) { return {s, s * 0.0625f, -1032.f * s, -72.f * s}; }
__device__ __forceinline__ float f16lo(uint32_t p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t p) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16)); }
// The 8 codes of one packed dword -> 8 bf16 values bf16_rne(q * s), in k order, as 4 pairs.
__device__ __forceinline__ u32x4 dequant8_mix(uint32_t w, const I4Mix& m) {
  // (v & mask) ^ c with c = 0x6400 in each half plus the code's top bit: the fp16 bits and
  // the XOR with 8 in one three-input bit operation
  const uint32_t y = w >> 8;
  const uint32_t p0 = (w & 0x000f000fu) ^ 0x64086408u;  // codes 0 (low half) and 4 (high half)
  const uint32_t p1 = (w & 0x00f000f0u) ^ 0x64806480u;  // codes 1 and 5, times 16
  const uint32_t p2 = (y & 0x000f000fu) ^ 0x64086408u;  // codes 2 and 6
  const uint32_t p3 = (y & 0x00f000f0u) ^ 0x64806480u;  // codes 3 and 7, times 16
  u32x4 o;
  o[0] = pack_bf16(fmaf(f16lo(p0), m.s, m.c0), fmaf(f16lo(p1), m.s16, m.c1));
  o[1] = pack_bf16(fmaf(f16lo(p2), m.s, m.c0), fmaf(f16lo(p3), m.s16, m.c1));
  o[2] = pack_bf16(fmaf(f16hi(p0), m.s, m.c0), fmaf(f16hi(p1), m.s16, m.c1));
  o[3] = pack_bf16(fmaf(f16hi(p2), m.s, m.c0), fmaf(f16hi(p3), m.s16, m.c1));
  return o;
}

// dequant8_mix in stages of two or three VALU operations (stage s after MFMA s of a row, s =
// 0..6), and the last pack (dequant8_mix_last) with the store after MFMA 7: the same operations
// on the same values, hence the same bits.
struct I4Stage {
  uint32_t y, p0, p1, p2, p3;
  u32x4 o;  // one vector, written element-wise: kept whole in registers
  float t0, t1;
};
__device__ __forceinline__ void dequant8_mix_stage(int s, uint32_t w, const I4Mix& m, I4Stage& t) {
  switch (s) {  // s is a constant after unrolling
    case 0:
      t.y = w >> 8;
      t.p0 = (w & 0x000f000fu) ^ 0x64086408u;
      t.p1 = (w & 0x00f000f0u) ^ 0x64806480u;
      break;
    case 1:
      t.t0 = fmaf(f16lo(t.p0), m.s, m.c0);
      t.t1 = fmaf(f16lo(t.p1), m.s16, m.c1);
      break;
    case 2:
      t.o[0] = pack_bf16(t.t0, t.t1);
      t.p2 = (t.y & 0x000f000fu) ^ 0x64086408u;
      t.p3 = (t.y & 0x00f000f0u) ^ 0x64806480u;
      break;
    case 3:
      t.t0 = fmaf(f16lo(t.p2), m.s, m.c0);
      t.t1 = fmaf(f16lo(t.p3), m.s16, m.c1);
      break;
    case 4:
      t.o[1] = pack_bf16(t.t0, t.t1);
      t.t0 = fmaf(f16hi(t.p0), m.s, m.c0);
      break;
    case 5:
      t.t1 = fmaf(f16hi(t.p1), m.s16, m.c1);
      t.o[2] = pack_bf16(t.t0, t.t1);
      break;
    case 6:
      t.t0 = fmaf(f16hi(t.p2), m.s, m.c0);
      t.t1 = fmaf(f16hi(t.p3), m.s16, m.c1);
      break;
    default:
      break;
  }
}
__device__ __forceinline__ u32x4 dequant8_mix_last(const I4Stage& t) {
  u32x4 r = t.o;
  r[3] = pack_bf16(t.t0, t.t1);
  return r;
}

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Store a wave's 128 x 128 block of an MFMA result as bf16 through a private 32 KB LDS
// buffer.  acc[i * 8 + j] holds output rows j*16 + (lane & 15) and columns i*16 + 4*(lane >> 4)
// .. +3 (the transposed-operand layout of the kernels).  Staging rows are 256 bytes with the
// 16-byte slot of chunk c at c ^ (row & 15), so both the 8-byte writes and the 16-byte
// reads are free of bank conflicts; each store instruction then writes four whole 256-byte
// row segments.  Rows >= rows_valid and columns >= cols_valid (a multiple of 8) are dropped.
__device__ __forceinline__ void store_block_bf16(const f32x4* acc, uint16_t* stage, uint16_t* out,
                                                 size_t ld, int rows_valid, int cols_valid,
                                                 int lane) {
  const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = 2 * i + (g4 >> 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = j * 16 + l16;
      const f32x4 v = acc[i * 8 + j];
      const u32x2 o = {pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      *reinterpret_cast<u32x2*>(stage + row * 128 + ((c ^ l16) << 3) + (g4 & 1) * 4) = o;
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes have landed
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    const int row = p * 4 + (lane >> 4), c = lane & 15;
    const u32x4 v = ld16(stage + row * 128 + ((c ^ (row & 15)) << 3));
    if (row < rows_valid && c * 8 < cols_valid) st16(out + (size_t)row * ld + c * 8, v);
  }
}

// ---- MXFP4: E2M1 codes in the int4 nibble layout, one E8M0 exponent per 32 k ----
// E2M1 pairs to bf16 with the block scale, on the gfx950 conversion instruction: byte `sel` of
// `codes` (low nibble first) becomes the low and high bf16 of the result, value * scale (exact
// here: at most two significant bits, normal exponents)
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t codes, float scale, int sel) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r;
  switch (sel) {  // the selector must be a constant
    case 0: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 0); break;
    case 1: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 1); break;
    case 2: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 2); break;
    default: r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, 3); break;
  }
  return __builtin_bit_cast(uint32_t, r);
}
// 8 codes (one dword, k ascending from the low nibble) to 8 bf16 in k order
__device__ __forceinline__ u32x4 dequant8_fp4(uint32_t codes, float scale) {
  return (u32x4){fp4x2_to_bf16x2(codes, scale, 0), fp4x2_to_bf16x2(codes, scale, 1),
                 fp4x2_to_bf16x2(codes, scale, 2), fp4x2_to_bf16x2(codes, scale, 3)};
}
// E8M0 exponent byte -> 2^(E - 127) (E in 1..254; the quantiser writes 2..252)
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) { return __uint_as_float(e << 23); }

// Workgroup id -> logical tile id such that each of the 8 XCDs (which receive workgroups
// round-robin by id) owns one contiguous range of logical tiles; a bijection for any total.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, rem = total & 7;
  const int x = bid & 7, local = bid >> 3;
  return x * q + min(x, rem) + local;
}

// Logical tile id -> (row tile, column tile), walking `group` row tiles at a time so that
// workgroups running together share operand panels in L2.
__device__ __forceinline__ void grouped_tile(int t, int tiles_r, int tiles_c, int group,
                                             int& tr, int& tc) {
  const int per = group * tiles_c;
  const int g = t / per;
  const int first = g * group;
  const int gs = min(group, tiles_r - first);
  const int r = t - g * per;
  tr = first + r % gs;
  tc = r / gs;
}

}  // namespace lora

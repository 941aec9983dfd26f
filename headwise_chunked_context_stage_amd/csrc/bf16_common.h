// bf16_common.h -- shared device helpers of the bf16 kernels for gfx950
// (CDNA4): MFMA wrapper, packing, XCD-aware workgroup order, and the LDS tile
// layout with its two conflict-free read patterns used by the attention
// kernels.  Included by each kernel source; everything has internal linkage.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace upipe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int DH = 128;  // head dimension of the bf16 path

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ bf16x8 frag(const u16* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Hardware exp2 (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> one dword of two bf16 (round to nearest even): v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// Registers 8t..8t+7 of a C block -> an 8-slot bf16 operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int t) {
  u32x4 r;
  r[0] = pack2(c[8 * t + 0], c[8 * t + 1]);
  r[1] = pack2(c[8 * t + 2], c[8 * t + 3]);
  r[2] = pack2(c[8 * t + 4], c[8 * t + 5]);
  r[3] = pack2(c[8 * t + 6], c[8 * t + 7]);
  return __builtin_bit_cast(bf16x8, r);
}


// Map a workgroup id so that each XCD (ids are dealt round-robin over 8 XCDs)
// runs one contiguous range of logical ids.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int x = id % 8, local = id / 8;
  const int per = total / 8, rem = total % 8;
  return x * per + min(x, rem) + local;
}

// Rounds of 256 consecutive workgroup ids (one per CU at a time): within a
// round, XCD x (ids are dealt round-robin over 8 XCDs) gets 32 consecutive
// logical ids, and the order of the XCDs reverses every other round, so each
// XCD's L2 serves neighbouring tiles while heavy and light tiles stay evenly
// spread over the XCDs.  A trailing partial round keeps the identity map.
__device__ __forceinline__ int xcd_snake(int id, int total) {
  const int round = id >> 8, pos = id & 255;
  if ((round << 8) + 256 > total) return id;
  const int x = pos & 7, j = pos >> 3;
  const int xx = (round & 1) ? 7 - x : x;
  return (round << 8) + xx * 32 + j;
}

// ================================================================= attention
// Tiles of 128-column bf16 rows live in LDS row-major with a padded row
// stride (RS = 136 elements, 272 bytes: consecutive physical rows start 4
// banks apart) and a fixed permutation of the rows inside every 16-row group:
// logical row 8a + 4b + c (a, b in {0,1}, c < 4) sits at physical row
// 4c + 2b + a.  Two read patterns are then free of bank conflicts and all
// their addresses are affine (immediate offsets):
//  * row operand (ds_read_b128): each lane reads 8 columns of its own row; 16
//    consecutive logical rows are 16 distinct physical rows;
//  * column operand (ds_read_b64_tr_b16): a 16-lane group reads 4 logical
//    rows 4b..4b+3 (physical rows four apart, 16 banks apart) x 32 bytes, so
//    the two groups of a half wave (columns 16 apart, 8 banks) interleave.
// The transposing read gives lane i of each 16-lane group element (i % 4) of
// the 8-byte rows addressed by lanes 4k + i/4 (k = 0..3).  When lane 4k + c of
// the group addresses row R_k at columns n0 + 4c .. n0 + 4c + 3, lane i
// receives column n0 + i of rows R_0..R_3: four k-slots of an MFMA operand
// whose lane index is a column of the tile.  Two such reads fill the 8 slots
// in the row order of a C block (rows 4h..4h+3, then 8+4h..8+4h+3 of each
// 16-row step), so they pair with P or dS taken from registers.
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int RS = DH + 8;  // LDS row stride of attention tiles (elements)

typedef __attribute__((address_space(3))) u16 lds_u16;

__device__ __forceinline__ int prow(int q) {
  return (q & ~15) | ((q & 3) << 2) | (((q >> 2) & 1) << 1) | ((q >> 3) & 1);
}

// Element offset of (logical row q, column col) in a tile.
__device__ __forceinline__ int toff(int q, int col) { return prow(q) * RS + col; }

// Per-lane base addresses of one tile for the two read patterns.  They are
// passed through an empty asm so the compiler keeps exactly one register per
// pattern and folds every fragment's constant offset into the instruction,
// instead of hoisting one address register per fragment out of the loop.
struct TileAddr {
  const lds_u16* row;  // + (32*blk)*RS + 16*t: row operand of rows 32*blk + lane%32, columns 16t + 8h..
  const lds_u16* col;  // + r0*RS + n0: column operand (first 4 slots; the other 4 are one row further)
};
__device__ __forceinline__ const lds_u16* opaque(const lds_u16* p) {
  unsigned v = static_cast<unsigned>(reinterpret_cast<uintptr_t>(p));
  asm volatile("" : "+v"(v));
  return reinterpret_cast<const lds_u16*>(static_cast<uintptr_t>(v));
}
__device__ __forceinline__ TileAddr tile_addr(const u16* tile, int lane) {
  const lds_u16* t = (const lds_u16*)tile;  // generic -> LDS address space
  const int hf = lane >> 5, g16 = (lane >> 4) & 1, i16 = lane & 15;
  TileAddr ta;
  ta.row = opaque(t + prow(lane & 31) * RS + 8 * hf);
  ta.col = opaque(t + prow(4 * hf + (i16 >> 2)) * RS + 16 * g16 + 4 * (i16 & 3));
  return ta;
}

// Row operand: row 32*blk + lane%32, columns 16t + 8h .. 16t + 8h + 7.
__device__ __forceinline__ bf16x8 row_frag(const TileAddr& ta, int blk, int t) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
                                        ta.row + 32 * blk * RS + 16 * t));
}

// Column operand: column n0 + lane % 32 of the 16 rows r0 .. r0 + 15 (r0 a
// multiple of 16), in the slot order of a C block (lane half h: rows
// r0+4h..r0+4h+3, then r0+8+4h..r0+8+4h+3; the second set is one physical row
// further).
__device__ __forceinline__ bf16x8 col_frag(const TileAddr& ta, int r0, int n0) {
  const lds_u16* p = ta.col + r0 * RS + n0;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lds_u16*>(p)));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) v4i16*>(const_cast<lds_u16*>(p + RS)));
  const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
  const u32x4 w = {l2[0], l2[1], h2[0], h2[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// One 256-byte row from global memory straight into LDS (no registers): lane
// l copies bytes 4l..4l+3 of the row at `src` to LDS byte address dst + 4l
// (global_load_lds_dword; M0 holds the LDS address).  `src` and `dst` are
// wave-uniform.  The copy is counted by vmcnt only and is not seen by the
// compiler's wait insertion: dma_wait() before the barrier that publishes the
// rows.  The kernels that use it issue no other global loads while copies are
// in flight, apart from the register path for tiles that run past S, whose
// compiler-inserted waits then cover the copies too.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_row(const void* src, unsigned dst, unsigned lane4) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(dst), "v"(lane4), "s"(src) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// max(x[l], x[l ^ 32]) in every lane l: v_permlane32_swap exchanges the two
// half-waves between two registers (both holding x), after which each lane
// holds its own value in one and its partner's in the other.  This stays in
// registers, where a 32-lane xor shuffle is an LDS permute round trip.
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// A register filled by a global load before a copy loop, made to arrive here.
// Because the wait insertion does not count the copies, a register still in
// flight where the loop starts gets an s_waitcnt vmcnt(0) before its first
// use in every iteration, and that wait also holds the wave until the copies
// it has just issued for the next tile have landed.  Waiting once, before the
// loop, keeps the loop free of it.
template <class T>
__device__ __forceinline__ void settle(T& x) {
  asm volatile("" : "+v"(x));
}
__device__ __forceinline__ unsigned lds_byte_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_u16*)p));
}

// ---- Swizzled attention tiles: 64 rows of 128 bf16 columns, 256-byte rows
// without padding; the 16-byte chunk c of row r sits at position c ^ swz(r),
// swz(r) = 4 (r % 4) + (r / 4) % 4.  Sixteen consecutive rows read at one
// chunk (row operands) and the transposing reads of four rows by 64 bytes
// (column operands) both touch every bank once per 256 bytes.  A tile can be
// filled by 4-row direct copies (global_load_lds_dwordx4: 1 KB of LDS per wave
// instruction), the lanes fetching their chunks from the permuted positions.
__device__ __forceinline__ int swz(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
struct SwzAddr {
  unsigned row;  // row operand, rows lane % 32 (+ 32 blk), chunk 2t + lane / 32: ^ 32t
  unsigned col;  // column operand, rows r0 + 4 (lane / 32) + (lane % 16) / 4, columns n0 + ...: ^ 64 (n0 / 32)
};
__device__ __forceinline__ SwzAddr swz_addr(const u16* tile, int lane) {
  const unsigned base = lds_byte_addr(tile);  // 256-byte aligned
  const int hf = lane >> 5, g16 = (lane >> 4) & 1, i16 = lane & 15, k = i16 >> 2, cp = i16 & 3;
  const int r0 = lane & 31;
  unsigned rw = base + r0 * 256u + 16u * (hf ^ swz(r0));
  unsigned cl = base + (4 * hf + k) * 256u + 64u * k + 16u * ((2 * g16 + (cp >> 1)) ^ hf) + 8u * (cp & 1);
  asm volatile("" : "+v"(rw), "+v"(cl));
  return SwzAddr{rw, cl};
}
__device__ __forceinline__ bf16x8 swz_row_frag(const SwzAddr& a, int blk, int t) {
  const unsigned p = (a.row ^ (32u * t)) + 8192u * blk;
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const lds_u32x4*>(static_cast<uintptr_t>(p)));
}
// Column operand: column n0 + lane % 32 of rows r0 .. r0 + 15 (r0 % 16 == 0,
// n0 % 32 == 0) in the slot order of a C block.
__device__ __forceinline__ bf16x8 swz_col_frag(const SwzAddr& a, int r0, int n0) {
  const unsigned lo = (a.col ^ (2u * n0)) + 256u * r0;
  const unsigned hi = (a.col ^ (2u * n0 + 32u)) + 256u * (r0 + 8);
  const v4i16 l4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16*>(static_cast<uintptr_t>(lo)));
  const v4i16 h4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_v4i16*>(static_cast<uintptr_t>(hi)));
  const u32x2 l2 = __builtin_bit_cast(u32x2, l4), h2 = __builtin_bit_cast(u32x2, h4);
  return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}
// Element offset of (row r, 16-byte chunk c) in a swizzled tile.
__device__ __forceinline__ int swz_off(int r, int c) { return r * 128 + 8 * (c ^ swz(r)); }
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// Rows 4q .. 4q + 3 (q < 4) of a 16-row block: src and dst are the block's
// first row (wave-uniform); voff = (lane / 16) * 256 + 16 ((lane % 16) ^ (4 (lane / 16) + q)).
__device__ __forceinline__ void dma_rows4(const void* src, unsigned dst, unsigned voff) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(dst), "v"(voff), "s"(src) : "memory", "m0");
}
#pragma clang diagnostic pop

// Copy rows [row0, row0 + nrows) of a [S][ld] bf16 matrix (128 columns from
// `src`) into a tile; rows at or beyond S are zero.  NCH chunks of 16 bytes
// per thread, thread t handling chunks t, t + 256, ...
template <int NCH, int NT = 256>
struct TileLoad {
  u32x4 r[NCH];
  __device__ __forceinline__ void load(const u16* src, int64_t ld, int64_t row0, int64_t S, int first) {
    constexpr int RSTEP = NT / 16;                // rows between a thread's chunks
    const int row = first >> 4, c = first & 15;  // rows row, row + RSTEP, ...
    const u16* p = src + (row0 + row) * ld + c * 8;
    const int64_t left = S - row0 - row;          // rows of this thread still inside S: m * RSTEP < left
#pragma unroll
    for (int m = 0; m < NCH; ++m) r[m] = RSTEP * m < left ? ld16(p + RSTEP * m * ld) : u32x4{0, 0, 0, 0};
  }
  __device__ __forceinline__ void store(u16* tile, int first) const {
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int e = first + NT * m, row = e >> 4, c = e & 15;
      st16(tile + toff(row, c * 8), r[m]);
    }
  }
};

}  // namespace
}  // namespace upipe

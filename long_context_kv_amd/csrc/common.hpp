// Shared device helpers for the cartridge-attention kernels (gfx950, wave64).
//
// MFMA operand convention used by every attention kernel here. For the
// 32x32 MFMAs (bf16 32x32x16 and f32 32x32x2) a wave holds:
//   A[i][k]  in lane (i + 32*kh), item t   with k = slot(kh, t)
//   B[k][j]  in lane (j + 32*kh), item t   with k = slot(kh, t)
//   D[i][j]  in lane (j + 32*h),  reg r    with i = (r & 3) + 4*h + 8*(r >> 2)
// where kh = lane / 32 and t < KPL (8 for bf16, 1 for f32). The kernels never
// depend on how the hardware orders slot(kh, t) inside one instruction: A and
// B are always filled from the same (kh, t) -> k map, so any order contracts
// the right pairs. The only layout fact used is the D map above, which lets
// the f32 result of one MFMA (rows = keys, columns = queries) be fed back as
// the B operand of the next one after a cast, with k = the key rows in the
// order row_of(r, h) = (r & 3) + 4*h + 8*(r >> 2).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace cartattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

// float -> storage type; the bf16 conversion rounds to nearest even.
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Row index of register r of a 32x32 MFMA result in lane half h.
__device__ __forceinline__ constexpr int d_row(int r, int h) {
  return (r & 3) + 4 * h + 8 * (r >> 2);
}

// Per-type MFMA policy: KPL = contraction elements per lane per
// instruction; KSTEP = 2*KPL elements per instruction.
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KPL = 8;
  static constexpr int KSTEP = 16;
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KPL = 1;
  static constexpr int KSTEP = 2;
  typedef float frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// KPL consecutive elements starting at p (16-byte aligned for bf16).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag load_frag(const T* p);
template <> __device__ __forceinline__ bf16x8 load_frag<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ __forceinline__ float load_frag<float>(const float* p) { return *p; }

// Item t of a fragment.
__device__ __forceinline__ float frag_get(bf16x8 f, int t) { return (float)f[t]; }
__device__ __forceinline__ float frag_get(float f, int) { return f; }

// Build the B/A fragment for MFMA number m of the PV-type contraction from
// the f32 result registers of a previous MFMA: items t <- regs m*KPL + t.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag pack_regs(const f32x16& s, int m);
template <> __device__ __forceinline__ bf16x8 pack_regs<bf16>(const f32x16& s, int m) {
  bf16x8 f;
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = (bf16)s[m * 8 + t];
  return f;
}
template <> __device__ __forceinline__ float pack_regs<float>(const f32x16& s, int m) {
  return s[m];
}

// Load 8 consecutive elements of type TS from global memory and convert to
// f32 (used for staging rows into LDS with an optional dtype change).
template <typename TS>
__device__ __forceinline__ void load8(const TS* p, float (&v)[8]);
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <> __device__ __forceinline__ void load8<bf16>(const bf16* p, float (&v)[8]) {
  const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int t = 0; t < 8; ++t) v[t] = (float)a[t];
}

// Store 8 f32 values as 8 consecutive elements of type T.
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);
template <> __device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, const float (&v)[8]) {
  bf16x8 a;
#pragma unroll
  for (int t = 0; t < 8; ++t) a[t] = (bf16)v[t];
  *reinterpret_cast<bf16x8*>(p) = a;
}

// Workgroups are dispatched round-robin over the 8 XCDs of an MI355X. Map the
// hardware block id to a logical id so that each XCD receives one contiguous
// range of logical ids (and therefore shares K/V and accumulators in its own
// L2).
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd;
  const int idx = bid / kXcd;
  const int q = nblocks / kXcd;
  const int r = nblocks % kXcd;
  return (xcd < r) ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// Sum over aligned groups of N lanes (N = 8 or 16) by DPP adds: swap lanes
// 1 apart, 2 apart, then mirror halves of 8 and of 16.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                             0xF, true));
}
template <int N>
__device__ __forceinline__ float row_sum(float x) {
  static_assert(N == 8 || N == 16, "row of 8 or 16 lanes");
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (N == 16) x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}

// Combine lane l with lane l ^ 32 by gfx950's v_permlane32_swap (a VALU
// lane swap; a shuffle would go through LDS and wait for it). Both lanes get
// the lower-half value first and the upper-half value second, so their
// results are bit-identical. Written as inline assembly with both registers
// as outputs (the compiler builtin's second result was dropped in codegen),
// with wait states around it for the VALU hazards.
__device__ __forceinline__ float2 halves_pair(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  return make_float2(a, b);
}
__device__ __forceinline__ float wave_max_halves(float x) {
  const float2 p = halves_pair(x);
  return fmaxf(p.x, p.y);
}
__device__ __forceinline__ float wave_sum_halves(float x) {
  const float2 p = halves_pair(x);
  return p.x + p.y;
}

}  // namespace cartattn

namespace cartattn {

// LDS transpose read (gfx950 ds_read_b64_tr_b16). Measured lane mapping:
// inside each group of 16 lanes, lane j receives, as item t (t = 0..3),
// element (j % 4) of the 8-byte word addressed by lane (j / 4 + 4 t) of the
// group. tr_col4 therefore has lane s of a group address
// M[r0 + s/4][c0 + 4*(s%4)], so that lane j of the group ends up with the
// column strip M[r0 + t][c0 + j], t = 0..3, of a row-major tile M.
typedef short tr_v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 tr_col4(const bf16* tile, int stride, int r0, int c0,
                                          int lane) {
  const int s = lane & 15;
  const bf16* p = tile + (r0 + (s >> 2)) * stride + c0 + 4 * (s & 3);
  const tr_v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) tr_v4i16*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace cartattn

namespace cartattn {

// ---- LDS tiles for the bf16 kernels -------------------------------------
// A tile of R rows x D bf16 (R a multiple of 8) is stored row by row in
// groups of 8 rows. Row j of a group starts phi(j) 16-byte chunks past its
// unpadded place, and groups are GRP bytes apart. The shifts are chosen for
// the two read patterns of the kernels, on an LDS of 64 four-byte banks:
//  * a 16-byte row fragment per lane, rows 16 i .. 16 i + 15 of one column
//    chunk per 16 lanes: the 16 rows start in 16 different chunk residues
//    (mod 16) of the bank space;
//  * a transpose read, 4 rows x 64 bytes per 32 lanes: the 4 rows of an
//    aligned group of 4 start in residues 4 apart, so their 16-dword windows
//    are disjoint.
// Rows 0-3 of a group take residues = 0 (mod 4), rows 4-7 residues = 1, and
// GRP = 2 (mod 4) chunks moves the next group to residues 2 and 3. Measured
// on gfx950 for D = 128 this gives about 222 B/clk per CU for row fragments
// and 178 B/clk for transpose reads, against 213 and 111 for a plain row
// padding of 24 elements (the best plain padding for both patterns at
// once). Every fragment address is a per-lane base plus a compile-time
// offset, since row offsets used as immediates are multiples of 8 rows.
template <int D>
struct Tile {
  static constexpr int RC = D / 8;   // 16-byte chunks of a row
  static constexpr int phi(int j) {
    int f = 0, used = 0;
    for (int r = 0;; ++r) {
      if ((r & 3) == 0) used = 0;
      while ((((RC * r + f) & 3) != (r >> 2)) || ((used >> ((RC * r + f) & 15)) & 1)) ++f;
      used |= 1 << ((RC * r + f) & 15);
      if (r == j) return f;
    }
  }
  // first chunk of row j (0..7) inside its group
  static constexpr int start(int j) { return RC * j + phi(j); }
  static constexpr int span() { return start(7) + RC; }
  static constexpr int GC = span() + ((2 - span() % 4) + 4) % 4;   // chunks per group
  static constexpr int GRP = 16 * GC;                              // bytes per group
  // start(j) for a run-time j in closed form (checked against start below)
  __host__ __device__ static constexpr int start_rt(int j) {
    return RC * j + 4 * (RC == 16 ? j : j >> 1) - 3 * (j >> 2);
  }
  static constexpr bool closed_form_ok() {
    for (int j = 0; j < 8; ++j)
      if (start_rt(j) != start(j)) return false;
    return true;
  }
  // byte offset of (row r, column col) in the tile
  __host__ __device__ static constexpr int off(int r, int col) {
    return (r >> 3) * GRP + 16 * start_rt(r & 7) + 2 * col;
  }
  // byte offset between rows r and r + rows8 (rows8 a multiple of 8)
  static constexpr int rows(int rows8) { return rows8 / 8 * GRP; }
  // Row and column chunk stored at chunk position pos of the tile; cc >= RC
  // marks padding.
  __host__ __device__ static inline void locate(int pos, int& row, int& cc) {
    // evaluated by the compiler (start() is a loop, kept off the GPU)
    constexpr int st[8] = {start(0), start(1), start(2), start(3),
                           start(4), start(5), start(6), start(7)};
    const int g = pos / GC;
    const int o = pos - g * GC;
    int j = 0, s = 0;
#pragma unroll
    for (int t = 1; t < 8; ++t)
      if (o >= st[t]) { j = t; s = st[t]; }
    row = 8 * g + j;
    cc = o - s;
  }
};
static_assert(Tile<128>::GC % 4 == 2 && Tile<64>::GC % 4 == 2, "group size");
static_assert(Tile<128>::closed_form_ok() && Tile<64>::closed_form_ok(), "row starts");
static_assert(Tile<128>::GRP == 2464 && Tile<64>::GRP == 1184, "tile layout");

// Elements of a tile of NROWS rows (a multiple of 8 elements).
template <int D, int NROWS>
constexpr int tile_elems() {
  static_assert(NROWS % 8 == 0, "tiles hold whole groups of 8 rows");
  return (NROWS / 8) * Tile<D>::GRP / 2;
}

// Asynchronous global->LDS copies use buffer loads with the LDS bit (MUBUF
// encoding): lane l of one instruction writes its 16 bytes to byte 16*l past
// the wave-uniform LDS address, and bytes at or past `bytes` of the buffer
// read as zero. (The FLAT-encoded global_load_lds form would also count
// against the LDS counter, which makes every later LDS wait a full drain.)
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
// The same from values read from lane 0: where the compiler cannot see that
// the base and size are wave-uniform (values carried across branches, or
// formed by vector instructions), a descriptor left in vector registers
// turns every load through it into a loop over distinct descriptors.
__device__ __forceinline__ buf_rsrc uniform_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return make_rsrc((const void*)(uintptr_t)((uint64_t)hi << 32 | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}
// Cache-policy operand of a buffer load coherent at device scope on gfx950
// (the SC1 bit: the load is served from beyond the XCD's L2).
constexpr int kCpolDevice = 16;
__device__ __forceinline__ void dma16(buf_rsrc r, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)voff, 0, 0, 0);
}
// The same with the LDS destination `off` bytes past `lds` (an offset into
// the object `lds` points to, so the compiler still knows what is written).
__device__ __forceinline__ void dma16_at(buf_rsrc r, uint32_t voff, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) char*)lds + off, 16, (int)voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4_at(buf_rsrc r, uint32_t voff, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) char*)lds + off, 4, (int)voff, 0, 0, 0);
}

// Per-lane source offsets of this wave's share of the asynchronous copy of
// a tile of NROWS rows x D bf16 (global rows rs_bytes bytes apart) into an
// LDS tile of tile_elems<D, NROWS>() elements laid out as Tile<D> describes:
// 1 KiB loads spread over the NWAVE waves of the workgroup, lane l of block
// blk = NWAVE k + wave writing chunk position 64 blk + l (lanes past the end
// of the tile in the last block are switched off). Computed once per
// kernel: off[k] = byte offset of this lane's chunk in the wave's k-th
// block, the same for every tile. Lanes whose 16 bytes fall on padding
// re-read chunk 0 of their row.
template <int D, int NROWS, int NWAVE = 4>
struct TileMap {
  static constexpr int CHUNKS = tile_elems<D, NROWS>() / 8;
  static constexpr int NBLK = (CHUNKS + 63) / 64;
  static constexpr int LAST = CHUNKS - 64 * (NBLK - 1);   // lanes of the last block
  static constexpr int NK = (NBLK + NWAVE - 1) / NWAVE;
  uint32_t off[NK];
  __device__ TileMap(int wave, int lane, uint32_t rs_bytes) {
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      int rr, cc;
      Tile<D>::locate((NWAVE * k + wave) * 64 + lane, rr, cc);
      off[k] = (uint32_t)rr * rs_bytes + (uint32_t)(cc < D / 8 ? cc : 0) * 16;
    }
  }
};

// Block k (0 <= k < NK) of this wave's share of the copy of a tile into
// `lds`, read through `r`, whose range ends with the tile's last row: chunks
// of rows past it (a partial tile) read as zeros, finite data the caller
// masks. Blocks that are whole for every wave are issued with all lanes on
// and no branch; only the tile's last block switches lanes off (a single
// condition mixing the wave-uniform block test with the lane test made the
// compiler mask and branch around every copy). k must be a compile-time
// constant after inlining.
template <int D, int NROWS, int NWAVE>
__device__ __forceinline__ void dma_block(const TileMap<D, NROWS, NWAVE>& m, int k, bf16* lds,
                                          buf_rsrc r, int wave, int lane) {
  using TM = TileMap<D, NROWS, NWAVE>;
  const int blk = k * NWAVE + wave;   // wave-uniform
  if (NWAVE * k + NWAVE - 1 < TM::NBLK - 1) {
    dma16(r, m.off[k], lds + blk * 512);
  } else if (blk < TM::NBLK - 1) {
    dma16(r, m.off[k], lds + blk * 512);
  } else if (blk == TM::NBLK - 1) {
    if (lane < TM::LAST) dma16(r, m.off[k], lds + blk * 512);
  }
}

// ---- LDS reads issued as inline assembly --------------------------------
// The compiler neither orders these after copies into LDS that are still in
// flight nor tracks their completion: the caller guarantees that no pending
// copy targets the bytes read, and waits with lds_wait<N>() (at most N LDS
// operations of the wave still pending) before using a result. They are used
// where a read of one ring stage must overlap a copy into another stage.
// `base` is a per-lane LDS byte address, OFF a compile-time byte offset.
// Register operands of these statements are float vectors: with integer
// vector operands this compiler loses all but the first element.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ f32x4 lds_read16(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  f32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF));
  return v;
}
// ds_read_b64_tr_b16 (lane mapping as in tr_col4).
template <int OFF>
__device__ __forceinline__ bf16x4 lds_tr4(uint32_t base) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  f32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(base), "n"(OFF));
  return __builtin_bit_cast(bf16x4, v);
}
// ds_write_b128 of a float vector (completion counted like the reads).
template <int OFF>
__device__ __forceinline__ void lds_write16(uint32_t base, f32x4 v) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(base), "v"(v), "n"(OFF));
}
template <int N>
__device__ __forceinline__ void lds_wait() {
  static_assert(N >= 0 && N < 16, "lgkmcnt is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%0)" : : "n"(N));
}
// After lds_wait: pass a value read by one of the helpers above through an
// empty volatile statement, so that every use of it (and any reuse of its
// registers) comes after the wait. Volatile statements keep their order.
__device__ __forceinline__ void lds_tie(f32x4& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void lds_tie(bf16x8& x) {
  f32x4 v = __builtin_bit_cast(f32x4, x);
  asm volatile("" : "+v"(v));
  x = __builtin_bit_cast(bf16x8, v);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Workgroup barrier that orders LDS only: outstanding global stores and
// atomics of the wave are not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup barrier for code whose LDS traffic is all explicitly waited for:
// LDS reads issued by the inline-assembly helpers (lds_wait) and copies into
// LDS (CART_WAIT_VMCNT). lds_barrier's release fence would also wait for
// every copy still in flight, including those of tiles needed only later;
// this one keeps them in flight. The scheduling barriers keep the compiler
// from moving any instruction across it.
__device__ __forceinline__ void lds_barrier_waited() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Wait until at most n of this wave's vector memory operations are pending
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14).
#define CART_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt((((n) & 15) | ((((n) >> 4) & 3) << 14)) | 0x0F70)

}  // namespace cartattn

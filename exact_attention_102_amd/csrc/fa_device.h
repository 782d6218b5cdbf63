// fa_device.h -- device-side building blocks shared by the forward and backward
// kernels for gfx950 (CDNA4): MFMA wrappers, the swizzled LDS tile layout with
// its row-fragment and transposed (column) fragment reads, cross-half row
// reductions, and the work-item mapping over the 8 XCDs.
//
// MFMA register layouts (v_mfma_f32_32x32x16_bf16, one wave64):
//   A (32 x 16): lane l holds A[l % 32][8 * (l / 32) + e], e = 0..7
//   B (16 x 32): lane l holds B[8 * (l / 32) + e][l % 32]
//   C (32 x 32): lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]
// Row-fragment reads (ds_read_b128) feed operands whose contraction index runs
// along a tile row (d for Q K^T); column-fragment reads (two ds_read_b64_tr_b16)
// feed operands whose contraction index runs down a tile column (the key index of
// V in P V, the query index of Q and dO in dS^T Q and P^T dO).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

namespace fa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same MFMA written so that its result lands in vector registers, for short-lived
// products that VALU work consumes (S and dP in the dK/dV kernels) in kernels whose
// long-lived accumulators fill the accumulation registers: there the compiler gives
// every MFMA the accumulation-register form, and each such result is then read back one
// register at a time.  The compiler does not see these statements as MFMAs, so each
// statement opens with s_nop 1: an MFMA must not read a register in the 2 wait states
// after a VALU instruction wrote it, and under register pressure the compiler refills
// operand registers with VALU moves (v_accvgpr_read of a value it parked in an
// accumulation register) right before the statement.  A chain starts with C = 0 as an
// inline constant and ends with the result wait inside the same statement: at least 12
// wait states before any instruction after the statement can read a result (s_nop 7 +
// s_nop 3 after the second MFMA of a pair, s_nop 7 + s_nop 4 after a single one).
// Dependent MFMAs of a chain (C = the previous D, same registers) issue back to back.
// Each statement runs one k-step of two products, d0 += a0 b0 and d1 += a1 b1; a chain
// has at least two k-steps (KK = head dim / 16 >= 4 here).
__device__ __forceinline__ void mfma32v_first(f32x16& d0, f32x16& d1, bf16x8 a0, bf16x8 b0, bf16x8 a1,
                                              bf16x8 b1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, 0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, 0"
      : "=&v"(d0), "=&v"(d1)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}
__device__ __forceinline__ void mfma32v_step(f32x16& d0, f32x16& d1, bf16x8 a0, bf16x8 b0, bf16x8 a1,
                                             bf16x8 b1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1"
      : "+v"(d0), "+v"(d1)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}
__device__ __forceinline__ void mfma32v_last(f32x16& d0, f32x16& d1, bf16x8 a0, bf16x8 b0, bf16x8 a1,
                                             bf16x8 b1) {
  asm volatile(
      "s_nop 1\n\t"
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
      "s_nop 7\n\t"
      "s_nop 3"
      : "+v"(d0), "+v"(d1)
      : "v"(a0), "v"(b0), "v"(a1), "v"(b1));
}
// k-step kk of KK of the pair (the first step starts from 0, the last ends with the wait)
__device__ __forceinline__ void mfma32v_kstep(int kk, int KK, f32x16& d0, f32x16& d1, bf16x8 a0, bf16x8 b0,
                                              bf16x8 a1, bf16x8 b1) {
  if (kk == 0)
    mfma32v_first(d0, d1, a0, b0, a1, b1);
  else if (kk == KK - 1)
    mfma32v_last(d0, d1, a0, b0, a1, b1);
  else
    mfma32v_step(d0, d1, a0, b0, a1, b1);
}
// One product alone (d += a b), same conventions.
__device__ __forceinline__ void mfma32v_kstep1(int kk, int KK, f32x16& d, bf16x8 a, bf16x8 b) {
  if (kk == 0)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  else if (kk == KK - 1)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 4" : "+v"(d) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// The C layout puts rows 8a + 4b + i (b = lane half) in register 4a + i.  Feeding
// an MFMA's A operand row R with tile row pi(R) makes lane half g, registers
// 8h + e hold tile rows 16h + 8g + e: eight consecutive rows per register octet,
// exactly the k-slice a following MFMA's B operand wants for lane half g.
__device__ __forceinline__ int pi_row(int R) {
  const int a = R >> 3, b = (R >> 2) & 1, i = R & 3;
  return ((a >> 1) << 4) + (b << 3) + ((a & 1) << 2) + i;
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles of bf16, W elements per row (row pitch 2W bytes, no padding).
// The 16-byte chunk c of row r is stored at chunk position c ^ swz(r).  Two read
// shapes exist (64 banks of 4 bytes):
//  * row fragments (ds_read_b128): 16 lanes read the same chunk of 16 distinct rows;
//  * transposed reads (ds_read_b64_tr_b16): 16 lanes read 4 consecutive rows x 32
//    contiguous bytes, a half-wave 4 rows x 64 bytes.  Measured on gfx950, these
//    slow down when the XOR flips the lowest chunk bit (it reorders the two 16-byte
//    halves of a 32-byte row segment).
// A tile read only one way gets the best swizzle for that shape; a tile read both
// ways gets a compromise (all measured with MFMA-fed read loops):
//  kRowOnly  swz = bit-reversal of r % 16: 16 rows on 16 bank groups.
//  kColOnly  swz = 4 (r % 4): the 4 rows of a transposed read in 4 quarters, lowest
//            chunk bit untouched.
//  kBoth     swz = 4 (r % 4) ^ 2 ((r / 8) % 2): transposed reads as kColOnly; row
//            fragments 2-way at worst.
// W = 64 packs two rows per 256-byte bank line and uses the analogous bits on r / 2;
// W = 32 (only the dS^T tile, written by rows and read transposed) uses 2 ((r/8)%2).
// Wider tiles (W a multiple of 128, up to 384) use the W >= 128 patterns on every group
// of 16 chunks.
// Every transposed-readable variant satisfies swz(r + 4) == swz(r) for r % 8 < 4,
// so a transposed fragment's second read (4 rows further down) reuses the first
// read's lane offset, and every variant depends only on r % 16.
enum TileMode { kBoth = 0, kRowOnly = 1, kColOnly = 2 };

template <int W, int MODE>
__device__ __forceinline__ int swz(int row) {
  if constexpr (W == 32) {
    return ((row >> 3) & 1) << 1;
  } else if constexpr (W == 64) {
    const int x = row >> 1;  // two rows share a bank line; x picks the 128-byte half's partner set
    if constexpr (MODE == kRowOnly) return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
    if constexpr (MODE == kColOnly) return (x & 1) << 2;
    return ((x & 1) << 2) ^ (((row >> 3) & 1) << 1);
  } else {
    if constexpr (MODE == kRowOnly) return ((row & 1) << 3) | (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
    if constexpr (MODE == kColOnly) return (row & 3) << 2;
    return ((row & 3) << 2) ^ (((row >> 3) & 1) << 1);
  }
}

template <int W, int MODE>
__device__ __forceinline__ int tile_off(int row, int col) {  // byte offset of element (row, col)
  return row * (2 * W) + ((((col >> 3) ^ swz<W, MODE>(row))) << 4) + ((col & 7) << 1);
}

// Per-lane LDS byte offsets for row fragments of a W-wide tile: rows R + pi(l % 32)
// (R a multiple of 32) at elements 16 kk + 8 (l / 32) .. +7.  The swizzle only
// depends on r % 16, so one register per chunk pattern covers every R: the row base
// and the chunk-pair above 16 (W = 256) become compile-time constants folded into
// the ds_read immediate.  refresh() hides the values from loop-invariant hoisting,
// which would otherwise materialise (and spill) one register per (buffer, row,
// chunk) combination.
template <int W, int MODE>
struct RowOffsets {
  static constexpr int NR = (W / 16) < 8 ? (W / 16) : 8;
  int rf[NR];
  __device__ __forceinline__ void init(int lane, bool plain = false) {
    const int rrow = plain ? (lane & 31) : pi_row(lane & 31);
#pragma unroll
    for (int kk = 0; kk < NR; ++kk) rf[kk] = tile_off<W, MODE>(rrow, kk * 16 + (lane >> 5) * 8);
  }
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int i = 0; i < NR; ++i) asm volatile("" : "+v"(rf[i]));
  }
  __device__ __forceinline__ bf16x8 row(const LDS char* tile, int R, int kk) const {
    return *(const LDS bf16x8*)(tile + R * (2 * W) + (kk / NR) * 256 + rf[kk % NR]);
  }
};

// Per-lane offsets for transposed fragments: lane l gets
// tile[r0 + 8 (l / 32) + e][32 db + l % 32], e = 0..7, r0 a multiple of 16.  Each
// ds_read_b64_tr_b16 takes, per group of 16 lanes, four row segments of 4 elements
// and hands lane i the four values of column i; lane j of the group supplies row
// j / 4, columns 4 (j % 4) .. +3.
template <int W, int MODE>
struct ColOffsets {
  static constexpr int NC = (W / 32) < 4 ? (W / 32) : 4;
  int cf[NC];
  __device__ __forceinline__ static int lane_off(int lane, int db) {
    const int crow = ((lane >> 5) << 3) + ((lane & 15) >> 2);
    const int ccol = (((lane >> 4) & 1) << 4) + ((lane & 3) << 2);
    return tile_off<W, MODE>(crow, db * 32 + ccol);
  }
  // cb0: a first 32-column block (a column window); col(.., db) then reads block cb0 + db
  __device__ __forceinline__ void init(int lane, int cb0 = 0) {
#pragma unroll
    for (int db = 0; db < NC; ++db) cf[db] = lane_off(lane, cb0 + db);
  }
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int i = 0; i < NC; ++i) asm volatile("" : "+v"(cf[i]));
  }
  __device__ __forceinline__ static bf16x8 read_at(const LDS char* p) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)p);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS s16x4*)(p + 4 * (2 * W)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
  __device__ __forceinline__ bf16x8 col(const LDS char* tile, int r0, int db) const {
    return read_at(tile + r0 * (2 * W) + (db / NC) * 256 + cf[db % NC]);
  }
  // run-time db: computes the lane offset (indexing cf would force it into scratch)
  __device__ __forceinline__ static bf16x8 col_dyn(const LDS char* tile, int r0, int db, int lane) {
    return read_at(tile + r0 * (2 * W) + lane_off(lane, db));
  }
};

// One direct-to-LDS copy instruction (buffer_load_dwordx4 ... lds): lane l reads 16
// bytes at rsrc.base + soff + voff and writes them to LDS at lds + 16 l (M0 holds
// the LDS base; the s_nop is the wait state the hardware needs between a scalar
// write of M0 and an LDS-DMA instruction reading it).  M0 is written inside the
// statement and declared clobbered; nothing else in these kernels uses M0 (no
// LDS-DMA builtins, GWS or indexed register moves; the compiled code holds M0 only
// in these statements), so the compiler's warning about clobbering a reserved
// register has nothing to break.  The base must not be passed as an "{m0}" operand:
// the compiler then writes M0 itself right before the statement, and its hazard
// recognizer cannot see the LDS-DMA load inside, so no wait state separates the two
// and the load may use the previous M0 -- an LDS address outside the tile, possibly
// outside the workgroup's allocation.  A build of that form faulted the GPU.
//
// It is issued from inline assembly on purpose.  Through the compiler builtins,
// either form (global_load_lds, buffer_load ... lds) damages the wait-count
// placement of every LDS fragment read in the kernel: the global form is
// FLAT-class, so LDS-side completions are modelled as out of order and each read
// waits for all outstanding ones (lgkmcnt(0)); the buffer form is tracked as an
// asynchronous LDS store that every later LDS read is assumed to alias, so each
// read also waits for the in-flight prefetch of the next tile (vmcnt).  Here the
// compiler does not see the copy; the kernels order it themselves: wait_tile()
// (vmcnt(0)) and a barrier before a tile is read, and a barrier (which drains
// outstanding LDS reads) before a buffer is refilled.  Compiler-placed vmcnt waits
// for its own loads only over-wait when these copies are outstanding (the counter
// retires in order), so they stay correct.
// s_waitcnt immediate (gfx9 encoding): vmcnt 0, expcnt 7, lgkmcnt 15 (only vmcnt waits)
constexpr int kWaitVmcnt0 = 0x0F70;
// s_waitcnt immediate for vmcnt(n), n < 64 (vmcnt bits 3:0 and 15:14)
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, unsigned voff, unsigned soff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(soff), "s"(lds)
               : "m0");
}

// Buffer resource for raw dword loads over [base, base + bytes): word 1 holds
// address bits 32..47 with stride 0; word 3 selects data format 32 (the field must
// be non-zero for untyped loads), no swizzle, no index.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, unsigned bytes) {
  const unsigned long long b = (unsigned long long)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)b);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

__device__ __forceinline__ unsigned lds_addr(const LDS void* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)p);
}

// Direct-to-LDS copy of a ROWS x W bf16 tile: each wave instruction moves 64 x 16
// bytes straight into 1 KB of contiguous LDS (lane l lands at base + 16 l),
// bypassing registers.  Lane l therefore fetches the global chunk that belongs at
// its LDS position under the swizzle.  Global rows are ld bytes apart (any
// multiple of 16) and only their first nvalid 16-byte chunks exist: lanes whose
// chunk lies beyond get an offset past the buffer's range, which the hardware's
// range check turns into zeros without a memory access (the zero padding of a head
// dim below W).  The per-lane byte offsets of the pieces are computed once (init)
// and kept opaque to the optimiser (refresh); each issue is then one VALU-free
// instruction with a wave-uniform (SGPR) row offset.  Tiles reaching past
// valid_rows take a slower path that clamps rows to the last valid one: the kernels
// mask such keys (-inf scores) and give such queries P = 0, so the duplicates never
// count.  The copy is asynchronous: wait_tile() (vmcnt) plus a barrier must precede
// reads.
constexpr unsigned kOutOfRange = 0x80000000u;  // above every buffer range used here (< 2^31 bytes)

template <int ROWS, int W, int NW, int MODE>
struct TileDMA {
  static constexpr int kPieces = ROWS * W * 2 / 1024;
  static_assert(ROWS * W * 2 % 1024 == 0, "tile must split into whole 1 KB pieces");
  // pieces i * NW + wave per wave; when NW does not divide kPieces (5-7 waves) the
  // last round is issued by the waves that have a piece left (a wave-uniform test)
  static constexpr int kPerWave = (kPieces + NW - 1) / NW;
  static constexpr bool kEven = kPieces % NW == 0;
  unsigned off[kPerWave];
  unsigned ld;      // global row pitch, bytes
  int nvalid;       // 16-byte chunks per global row

  __device__ __forceinline__ static int piece_row(int piece, int lane) { return (piece * 1024 + lane * 16) / (2 * W); }
  __device__ __forceinline__ static int piece_chunk(int piece, int lane) {
    const int byte = piece * 1024 + lane * 16;
    return ((byte % (2 * W)) >> 4) ^ swz<W, MODE>(byte / (2 * W));
  }
  __device__ __forceinline__ static bool has(int i, int wave) { return kEven || i * NW + wave < kPieces; }
  // row_pitch_elems: the view's row stride (elements); head_dim: its valid columns
  __device__ __forceinline__ void init(int wave, int lane, long long row_pitch_elems, int head_dim) {
    ld = (unsigned)row_pitch_elems * 2u;
    nvalid = head_dim >> 3;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int piece = i * NW + wave;
      const int ch = piece_chunk(piece, lane);
      off[i] = ch < nvalid ? (unsigned)piece_row(piece, lane) * ld + (unsigned)ch * 16u : kOutOfRange;
    }
  }
  __device__ __forceinline__ void refresh() {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) asm volatile("" : "+v"(off[i]));
  }
  // wave must be wave-uniform (e.g. readfirstlane of threadIdx.x / 64); g is the
  // head's base and valid_rows its row count (valid_rows * ld < 2^31 bytes, so every
  // offset fits the 32-bit buffer range, which also bounds the reads).
  __device__ __forceinline__ void issue(const __bf16* g, int row0, int valid_rows, LDS char* tile, int wave,
                                        int lane) const {
    const u32x4 rs = buffer_rsrc(g, (unsigned)valid_rows * ld);
    if (row0 + ROWS <= valid_rows) {
      const unsigned soff = __builtin_amdgcn_readfirstlane((unsigned)row0 * ld);
#pragma unroll
      for (int i = 0; i < kPerWave; ++i)
        if (has(i, wave)) lds_dma16(rs, off[i], soff, lds_addr(tile + (i * NW + wave) * 1024));
    } else {
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        if (!has(i, wave)) continue;
        const int piece = i * NW + wave;
        const int grow = min(row0 + piece_row(piece, lane), valid_rows - 1);
        const int ch = piece_chunk(piece, lane);
        lds_dma16(rs, ch < nvalid ? (unsigned)grow * ld + (unsigned)ch * 16u : kOutOfRange, 0u,
                  lds_addr(tile + piece * 1024));
      }
    }
  }
};

// 16-byte register load of chunk `chunk` of a row (zeros past the head dim).
__device__ __forceinline__ bf16x8 load_row_chunk(const __bf16* row, int chunk, int nvalid) {
  if (chunk < nvalid) return *(const bf16x8*)(row + chunk * 8);
  bf16x8 z;
#pragma unroll
  for (int e = 0; e < 8; ++e) z[e] = (__bf16)0.f;
  return z;
}

// vmcnt(0) through the builtin (not inline assembly), so the compiler's own
// wait-count tracking also learns that all of its vector-memory loads are done.
__device__ __forceinline__ void wait_tile() { __builtin_amdgcn_s_waitcnt(kWaitVmcnt0); }

// Scheduling fence every CH iterations of an unrolled loop: bounds how many LDS
// fragment reads the scheduler hoists ahead of their MFMAs (each costs 4 VGPRs).
template <int CH>
__device__ __forceinline__ void fence_every(int i) {
  if (((i + 1) % CH) == 0) __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------
// Writes one wave's 32 x 32 DB fp32 accumulator tile to global memory as whole row
// segments.  In the C layout lane l holds row l % 32, columns 32 db + 8 a + 4 (l / 32)
// + 0..3 (registers 4 a .. 4 a + 3 of acc[db]), so a direct store instruction writes
// 32 rows x 32 bytes; staged through the wave's own LDS region (REGION bytes, free of
// any other use), each store instruction instead writes 64 / CPR complete row segments
// of CP columns.  Chunk c of row r sits at chunk position c ^ (r & SW) in the region (no
// bank conflicts beyond the 4 cycles a 1 KB access takes either way).  The region is
// reused pass by pass: the wave's LDS accesses complete in issue order.  Every value is
// multiplied by its row's factor (scale, one per lane).  row0 (wave-uniform) is the
// first row; rows from nrows on and columns from hd on are not written: lanes are
// masked.  The buffer range (nrows rows) does not do it alone -- a version that relied
// on it wrote rows past nrows, so the range check does not cover the scalar offset that
// selects a store's rows.  Offsets are 32-bit (the 32 rows span less than 2^31 bytes).
template <int DB, int REGION>
__device__ __forceinline__ void store_tile_rows(const f32x16 (&acc)[DB], float scale, LDS char* region, float* row0,
                                                long long sn, int nrows, int hd, int lane) {
  constexpr int CAP = REGION / (32 * 4);  // columns of 32 rows the region holds
  static_assert(CAP >= 32, "the staging region must hold 32 rows of 32 columns");
  constexpr int CP = CAP >= 128 ? 128 : CAP >= 64 ? 64 : 32;  // columns per pass
  constexpr int CPR = CP / 4;                                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                               // rows per store instruction
  constexpr int SW = CPR < 16 ? CPR - 1 : 15;
  constexpr int BPP = CP / 32;  // 32-column blocks per pass
  const int l32 = lane & 31, g = lane >> 5;
  const unsigned pitch = (unsigned)sn * 4u;  // bytes per row
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(row0, (short)0, (int)(nrows > 0 ? (unsigned)nrows * pitch : 0u), 0x00020000);
  const int rl = lane / CPR, c = lane % CPR;  // the lane's row within a store, its chunk
  const unsigned voff = (unsigned)rl * pitch + (unsigned)c * 16u;
#pragma unroll
  for (int p = 0; p < (DB + BPP - 1) / BPP; ++p) {
#pragma unroll
    for (int b = 0; b < BPP; ++b) {
      const int db = p * BPP + b;
      if (db < DB) {
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int cw = 8 * b + 2 * a4 + g;
          const f32x4 v = {acc[db][4 * a4] * scale, acc[db][4 * a4 + 1] * scale, acc[db][4 * a4 + 2] * scale,
                           acc[db][4 * a4 + 3] * scale};
          *(LDS f32x4*)(region + l32 * (CP * 4) + ((cw ^ (l32 & SW)) << 4)) = v;
        }
        __builtin_amdgcn_sched_barrier(0);  // one block's values at a time (register pressure)
      }
    }
    const int col = p * CP + 4 * c;
    const bool live = col < hd && col < 32 * DB;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + rl;
      const f32x4 v = *(const LDS f32x4*)(region + r * (CP * 4) + ((c ^ (r & SW)) << 4));
      if (live && r < nrows)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, voff + (unsigned)(p * CP * 4),
                                               (int)((unsigned)(RPI * i) * pitch), 0);
    }
  }
}

// ---------------------------------------------------------------------------
// Reductions across the two 32-lane halves (lane l and lane l ^ 32), which hold
// the two halves of a 32-key (or 32-query) block in the C layout.
__device__ __forceinline__ float half_swap_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + sum of the 8 bf16 values, accumulated in fp32 (v_dot2c_f32_bf16 against 1.0).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bf16x2 pr = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, acc, false);
  }
  return acc;
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& v, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[base + e];
  return r;
}

// ---------------------------------------------------------------------------
// Work-item mapping.  Workgroups are dispatched round-robin over the 8 XCDs
// (workgroup x lands on XCD x % 8), each with its own L2.  Remapping so that
// every XCD walks a contiguous range of work items keeps the tiles of one
// (batch, head) -- which all re-read the same K/V or Q/dO -- in one L2.
__device__ __forceinline__ int xcd_remap(int x, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = x & 7, local = x >> 3;
  return (xcd < r) ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Causal work order.  Tile costs differ (a query tile late in the sequence sees
// many keys; a key tile early in the sequence is seen by many queries), so the
// heaviest tiles are dispatched first.  With B*H a multiple of 8, XCD x (the one
// receiving workgroups x, x + 8, ...) keeps the heads h = x (mod 8) and walks
// them rank by rank, heaviest rank first; otherwise the order is rank-major over
// all heads.  heavy_high: the heaviest tile has the largest index.
__device__ __forceinline__ void causal_order(int x, int BH, int ntiles, bool heavy_high, int& bh, int& tile) {
  int rank;
  if ((BH & 7) == 0) {
    const int hp = BH >> 3, u = x >> 3;
    rank = u / hp;
    bh = (x & 7) + 8 * (u % hp);
  } else {
    rank = x / BH;
    bh = x % BH;
  }
  tile = heavy_high ? ntiles - 1 - rank : rank;
}

}  // namespace fa

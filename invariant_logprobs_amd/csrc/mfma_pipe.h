// mfma_pipe.h — pieces shared by the MFMA tile kernels of libtim.so
// (lmhead.hip, bwd.hip): operand types, the LDS ring geometry and swizzle,
// the buffer-to-LDS copy, the fragment reads and the wait helpers.  A tile
// kernel stages 256-row operand tiles of 128 bytes of K per pipeline stage
// through a five-position LDS ring and feeds MFMAs from it: 16x16x32 bf16 in
// the eight-wave kernels (the head's bf16 path, the backward's GEMMs),
// 32x32x2 fp32 in the head's four-wave fp32 kernel.
#pragma once

#include "tim_internal.h"

namespace tim {
namespace mfma {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// LDS: a ring of five positions, each holding one operand tile of a
// pipeline stage: 256 rows (W or h) of kStageBytes (128) per row, i.e. 64
// bf16 or 32 fp32 of K, four MFMA k-steps.  Tiles are filled by
// buffer_load_dwordx4 ... lds (64 lanes x 16 bytes = 8 rows of 128 bytes per
// instruction) one (W) or two (h) stages ahead of the MFMAs.  The eight
// 16-byte chunks of a row are XOR-swizzled with (row >> 1) & 7: the 16 lanes
// of one ds_read_b128 phase read 16 consecutive rows at one logical chunk,
// and with 128-byte rows those land on 16 distinct 16-byte bank groups of
// the 64-bank LDS.
constexpr int kPos = 5;                               // ring positions, one operand tile each
constexpr int kOperandBytes = kTileV * kStageBytes;   // 32 KiB
constexpr int kLdsBytes = kPos * kOperandBytes;       // 160 KiB
constexpr int kDmaPerStage = 16;                      // per wave: 8 W + 8 h blocks
static_assert(kTileV == kTileT, "one staging loop serves both operands");
static_assert(kStageBytes == 128, "swizzle and fragment mapping assume 128-byte rows");

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * kStageBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a raw buffer (base and size in the descriptor) at
// voffset + soffset, written to LDS at l + 16 * lane.  The row offsets are
// per lane and fixed; the K offset of a stage is the scalar soffset.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, void* l, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)l, 16, voff, soff, 0, 0);
}
constexpr int kRsrcWord3 = 0x00020000;   // buffer descriptor word 3: 32-bit data format,
                                         // no swizzle, no thread-id add

// Eight 16-byte LDS reads issued in one asm block, not waited for.  The ring
// is filled by LDS DMA; written as ordinary loads, the compiler cannot tell
// the slot being read from the slots still being filled and waits for every
// copy in flight (vmcnt(0)) before each read, which would serialise the
// pipeline.  The explicit vmcnt waits and barriers of the main loop order
// these reads after the copies of their stage; frags_ready() below waits for
// the reads themselves.  Outputs are early-clobber: a read's destination must
// not overlap a later read's address.
__device__ __forceinline__ void lds_issue_8x16(u32x4 (&r)[8], uint32_t aA, uint32_t aB) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:4096\n\t"
        "ds_read_b128 %2, %8 offset:8192\n\t"
        "ds_read_b128 %3, %8 offset:12288\n\t"
        "ds_read_b128 %4, %9\n\t"
        "ds_read_b128 %5, %9 offset:4096\n\t"
        "ds_read_b128 %6, %9 offset:8192\n\t"
        "ds_read_b128 %7, %9 offset:12288"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
          "=&v"(r[7])
        : "v"(aA), "v"(aB)
        : "memory");
}

// Wait until at most N LDS operations are outstanding; the fragments are
// passed through so that no use of them can be scheduled before the wait.
// LDS operations of a wave complete in order, so with the 8 reads of the
// other fragment set issued later, lgkmcnt(8) means this set has arrived.
template <int N>
__device__ __forceinline__ void frags_ready(u32x4 (&f)[8]) {
    static_assert(N == 0 || N == 8, "lgkmcnt values used here");
    if constexpr (N == 0)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]),
                       "+v"(f[6]), "+v"(f[7]));
    else
        asm volatile("s_waitcnt lgkmcnt(8)"
                     : "+v"(f[0]), "+v"(f[1]), "+v"(f[2]), "+v"(f[3]), "+v"(f[4]), "+v"(f[5]),
                       "+v"(f[6]), "+v"(f[7]));
}

// 16x16x32 pipeline.  One 16-byte LDS read per fragment, issued alone (the
// immediate offset selects the 16-row block), not waited for; wait16<N>
// waits until at most N LDS operations are outstanding and passes the
// fragments that the next MFMAs read through the asm, so that no use of
// them can be scheduled before the wait.  It ends with one wait state, as
// the compiler places between such a wait and an MFMA reading its result.
template <int kOff>
__device__ __forceinline__ void lds_read16(u32x4& r, uint32_t addr) {
    static_assert(kOff >= 0 && kOff < 65536, "ds_read immediate offset");
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff) : "memory");
}
template <int N>
__device__ __forceinline__ void wait16(u32x4& a) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%1)\n\ts_nop 0" : "+v"(a) : "i"(N));
}
template <int N>
__device__ __forceinline__ void wait16(u32x4& a, u32x4 (&b)[8]) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%9)\n\ts_nop 0"
                 : "+v"(a), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]), "+v"(b[4]),
                   "+v"(b[5]), "+v"(b[6]), "+v"(b[7])
                 : "i"(N));
}

// A fragment of an operand stored K-major ([K][M], M contiguous) in LDS:
// two transposing reads (ds_read_b64_tr_b16), K elements 0-3 and 4-7 of the
// lane's eight, written into the two halves of one 128-bit fragment.
// Within each 16-lane group, lane i receives element (i & 3) of the 8-byte
// row addressed by lane (i >> 2) + 4 j as its element j, so lane p of the
// group addresses K row (p >> 2) of its four at M offset 4 (p & 3): lane i
// then holds M = i, K = j of the group's four rows, the layout of a
// 16x16x32 MFMA source (row l & 15, K 8 (l >> 4) + 0..7).  The halves are
// outputs of the asm (so not waited for, like lds_read16's) that the
// register allocator places as the two halves of the fragment's register
// tuple; a copy in between would read them before their wait, which the
// library's code check rules out.
template <int kOff>
__device__ __forceinline__ void lds_read_tr(u32x4& r, uint32_t addr) {
    static_assert(kOff >= 0 && kOff + 2048 < 65536, "ds_read immediate offset");
    u32x2 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(addr), "i"(kOff) : "memory");
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(hi) : "v"(addr), "i"(kOff + 2048) : "memory");
    r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3);
}

template <int N>
__device__ __forceinline__ void wait16_4(u32x4& a, u32x4 (&b)[4]) {
    static_assert(N >= 0 && N <= 15, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%5)\n\ts_nop 0"
                 : "+v"(a), "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3])
                 : "i"(N));
}

// 16x16x32 bf16 MFMA with the accumulator tied (the same AGPRs are source C
// and destination).  With the builtin, and every accumulator register
// taken, the register allocator picked untied forms and shuffled
// accumulators between registers inside the K loops.  The hazard recognizer
// does not look into asm: the kernels place these so that the wait states
// it would insert are there anyway (the first MFMA of a tile follows its
// accumulator writes by more than the two wait states a VALU write needs:
// the loop opens with four LDS reads and a wait), and the stage's last MFMA
// is mfma16_tied_last below.
__device__ __forceinline__ void mfma16_tied(f32x4& acc, const u32x4& a, const u32x4& b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// The same, followed when `last` (an SGPR value) is non-zero by 20 wait
// states, more than the 19 that the longest case needs between an MFMA and a
// read of its result: the last MFMA of a tile.  MFMAs complete in issue
// order, so after it every accumulator may be read.  One asm statement:
// nothing the compiler places after the loop (a copy, a spill) can come
// between.  (A separate wait after the loop let such code in; peeling the
// last stage, or a wait taking every accumulator as an operand, made the
// register allocator copy accumulators inside the loop.)
__device__ __forceinline__ void mfma16_tied_last(f32x4& acc, const u32x4& a, const u32x4& b,
                                                 int last) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0\n\t"
                 "s_cmp_eq_u32 %3, 0\n\t"
                 "s_cbranch_scc1 .Lmfma_no_wait%=\n\t"
                 "s_nop 7\n\ts_nop 7\n\ts_nop 3\n"
                 ".Lmfma_no_wait%=:"
                 : "+a"(acc) : "v"(a), "v"(b), "s"(last) : "scc");
}

// The wait after the last of a sequence of tied asm MFMAs on acc[8][NB]:
// 20 wait states, more than any MFMA result needs before another instruction
// reads it, with every accumulator block an operand so that no read of one
// can be placed before it.  For the small accumulator sets of the narrow
// kernels (NB = 1, 2, 4).
template <int NB>
__device__ __forceinline__ void mfma_drain(f32x4 (&acc)[8][NB]);
template <>
__device__ __forceinline__ void mfma_drain<1>(f32x4 (&a)[8][1]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+a"(a[0][0]), "+a"(a[1][0]), "+a"(a[2][0]), "+a"(a[3][0]), "+a"(a[4][0]),
                   "+a"(a[5][0]), "+a"(a[6][0]), "+a"(a[7][0]));
}
// Four blocks: the wait in a first statement that takes blocks 0 and 1 of
// every row, a second (empty) one taking blocks 2 and 3 right after it (an
// asm statement takes at most 30 operands); volatile statements keep their
// order, so no read of any block comes before the wait.
template <>
__device__ __forceinline__ void mfma_drain<4>(f32x4 (&a)[8][4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+a"(a[0][0]), "+a"(a[1][0]), "+a"(a[2][0]), "+a"(a[3][0]), "+a"(a[4][0]),
                   "+a"(a[5][0]), "+a"(a[6][0]), "+a"(a[7][0]), "+a"(a[0][1]), "+a"(a[1][1]),
                   "+a"(a[2][1]), "+a"(a[3][1]), "+a"(a[4][1]), "+a"(a[5][1]), "+a"(a[6][1]),
                   "+a"(a[7][1]));
    asm volatile(""
                 : "+a"(a[0][2]), "+a"(a[1][2]), "+a"(a[2][2]), "+a"(a[3][2]), "+a"(a[4][2]),
                   "+a"(a[5][2]), "+a"(a[6][2]), "+a"(a[7][2]), "+a"(a[0][3]), "+a"(a[1][3]),
                   "+a"(a[2][3]), "+a"(a[3][3]), "+a"(a[4][3]), "+a"(a[5][3]), "+a"(a[6][3]),
                   "+a"(a[7][3]));
}
template <>
__device__ __forceinline__ void mfma_drain<2>(f32x4 (&a)[8][2]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+a"(a[0][0]), "+a"(a[1][0]), "+a"(a[2][0]), "+a"(a[3][0]), "+a"(a[4][0]),
                   "+a"(a[5][0]), "+a"(a[6][0]), "+a"(a[7][0]), "+a"(a[0][1]), "+a"(a[1][1]),
                   "+a"(a[2][1]), "+a"(a[3][1]), "+a"(a[4][1]), "+a"(a[5][1]), "+a"(a[6][1]),
                   "+a"(a[7][1]));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt vmcnt(N) only (gfx9 encoding; expcnt and lgkmcnt fields at max)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <bool B> struct BoolConst { static constexpr bool value = B; };
template <int I> struct IntConst { static constexpr int value = I; };

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

}  // namespace mfma
}  // namespace tim

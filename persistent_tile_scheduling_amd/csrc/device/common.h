// Device-side helpers shared by every kernel of the library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pts {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define PTS_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

// Compile-time loop: f(IntC<0>{}), ..., f(IntC<N-1>{}), so each step can use
// its index as a template argument (an instruction immediate).
template <int I> struct IntC {
    static constexpr int value = I;
};
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(IntC<I>{});
        static_for<N, I + 1>(f);
    }
}

// s_waitcnt immediate for the gfx9 family: vmcnt[3:0] in bits 3:0, expcnt in
// bits 6:4, lgkmcnt in bits 11:8, vmcnt[5:4] in bits 15:14. A field at its
// maximum means "do not wait on this counter".
constexpr int waitcnt_imm(int vm, int exp, int lgkm)
{
    return (vm & 0xF) | ((exp & 0x7) << 4) | ((lgkm & 0xF) << 8) | (((vm >> 4) & 0x3) << 14);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
// Vector-memory loads (including global->LDS loads) complete in issue order,
// so this waits for all but the N youngest loads.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 7, 15));
}

// Wait for this wave's outstanding LDS operations (and scalar loads).
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 7, 0));
}

__device__ __forceinline__ void wait_all()
{
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0, 0));
}

// Workgroup barrier. The "memory" clobber keeps the compiler from moving
// memory accesses across it; the hardware ordering of LDS and vector-memory
// traffic is the caller's job (explicit waits before the barrier). This is
// used instead of __syncthreads(), whose fence would also wait for every
// outstanding global->LDS load and so serialize the load pipeline.
__device__ __forceinline__ void barrier_raw()
{
    asm volatile("s_barrier" ::: "memory");
}

// LDS-visible barrier: this wave's LDS writes complete, then all waves meet.
__device__ __forceinline__ void barrier_lds()
{
    wait_lgkmcnt0();
    barrier_raw();
}

// Raw buffer descriptor (gfx9 layout) over `base`: no stride, no swizzle,
// 32-bit data format, and a record count that disables range clamping (the
// offsets this library forms always stay inside the operand).
__device__ __forceinline__ u32x4 buffer_rsrc(const void *base)
{
    const uint64_t b = (uint64_t)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
    r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xFFFFu);
    r[2] = 0xFFFFFFFFu;
    r[3] = 0x00020000u;
    return r;
}

// One wave-wide 16-byte-per-lane global -> LDS load: lane l's 16 bytes from
// buffer offset voff + soff land at LDS byte lds_addr + 16 l.
//
// Written as inline assembly on purpose: the compiler tracks its own LDS-DMA
// builtins as LDS writes that may alias any later LDS read, and then inserts
// vector-memory waits before the fragment reads of OTHER ring stages, which
// serializes the prefetch. Here the kernel alone accounts for these loads
// (explicit vmcnt waits before each stage is read). M0 carries the LDS
// destination. M0 is a reserved register the compiler sets itself before each
// instruction of its own that reads it, so it is not named as clobbered (the
// compiler warns that a reserved register in a clobber list is not honoured).
__device__ __forceinline__ void dma_load16(uint32_t lds_addr, uint32_t voff, u32x4 rsrc, uint32_t soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff)
                 : "memory");
}

// The same load with its LDS destination given as a scalar base plus a
// compile-time byte offset, added straight into M0 (one instruction where a
// copy and an add would otherwise precede the M0 write).
template <int LDS_IMM>
__device__ __forceinline__ void dma_load16_at(uint32_t lds_base, uint32_t voff, u32x4 rsrc, uint32_t soff)
{
    asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff), "i"(LDS_IMM)
                 : "memory", "scc");
}

// dma_load16_at with the byte offset as an argument: `lds_imm` must fold to a
// constant by code generation (a literal, or the index of a fully unrolled
// loop); the compiler rejects the statement otherwise.
__device__ __forceinline__ void dma_load16_imm(uint32_t lds_base, int lds_imm, uint32_t voff, u32x4 rsrc,
                                               uint32_t soff)
{
    asm volatile("s_add_u32 m0, %0, %4\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(lds_base), "v"(voff), "s"(rsrc), "s"(soff), "i"(lds_imm)
                 : "memory", "scc");
}

// The same load, performed only when `on` (a wave-uniform flag): with `on`
// false the load runs with no lanes enabled, so it neither reads memory nor
// writes LDS. Used where a branch around the load would cost more than the
// load itself. EXEC is restored before the statement ends; the wave's EXEC
// must be all ones here (the callers run uniformly).
__device__ __forceinline__ void dma_load16_if(uint32_t lds_addr, uint32_t voff, u32x4 rsrc, bool on)
{
    const uint32_t m = __builtin_amdgcn_readfirstlane(on ? 0xFFFFFFFFu : 0u);
    const uint64_t mask = ((uint64_t)m << 32) | m;
    uint64_t saved;
    asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, %5\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved)
                 : "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(0u), "s"(mask)
                 : "memory");
}

// The lanes of one wave exchange data through LDS here: each reads back what
// other lanes wrote. The compiler models lanes as threads that do not see each
// other's unsynchronized writes, so without this it may reuse a lane's earlier
// load of an address the lane itself did not write in between (and it did,
// moving reads into a branch only some lanes took). A wave performs its own
// LDS operations in order, so no instruction is needed, only the compiler
// barrier.
__device__ __forceinline__ void wave_lds_exchange()
{
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_address(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// 100 MHz constant-rate device clock, comparable across compute units.
__device__ __forceinline__ uint64_t realtime()
{
    return __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ uint32_t hw_id_reg()
{
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(v));
    return v;
}

// Shader (core) clock counter; with realtime() it gives the clock frequency.
__device__ __forceinline__ uint64_t shader_cycles() { return __builtin_amdgcn_s_memtime(); }

__device__ __forceinline__ uint32_t xcc_id_reg()
{
    uint32_t v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    return v & 0xF;
}

// Hide a value's origin from the optimizer so that expressions built on it
// are recomputed where used instead of being hoisted out of the persistent
// loop (where dozens of hoisted addresses would occupy registers for the whole
// kernel). "s" keeps it in a scalar register, "v" in a vector register.
__device__ __forceinline__ uint32_t opaque_s(uint32_t v)
{
    asm volatile("" : "+s"(v));
    return v;
}

__device__ __forceinline__ uint32_t opaque_v(uint32_t v)
{
    asm volatile("" : "+v"(v));
    return v;
}

// This lane's index in the wave (0..63), computed afresh from the exec mask
// (which must be all ones): nothing holds it in a register between uses, and
// the compiler cannot merge two computations of it into one long-lived value.
__device__ __forceinline__ uint32_t lane_id()
{
    uint32_t v;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(v));
    return v;
}

__device__ __forceinline__ int uniform(int v)
{
    return __builtin_amdgcn_readfirstlane(v);
}

} // namespace pts

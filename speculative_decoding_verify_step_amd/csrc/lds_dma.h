// lds_dma.h -- direct global -> LDS copies and the waits that go with them.
#pragma once
#include "common.h"

// The global -> LDS copies are issued from inline assembly: the compiler
// then does not treat them as pending writes to every LDS location (it would
// wait for all of them, the stages still in flight included, before any LDS
// read).  They have no register results; the waits for them are explicit:
// s_waitcnt vmcnt <= N, and a workgroup barrier, both also compiler barriers
// for memory accesses.
template <int N>
SV_DEV void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
SV_DEV void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// the same after this wave's LDS reads have completed (before a slot they
// read from is refilled by another wave's copy)
SV_DEV void lds_read_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// 16 bytes per lane from global memory to LDS at lds_off + 16 * lane.  The
// copy takes its LDS address from M0, which the compiler reserves: it is
// saved and restored around the copy, and the copy waits one state after M0
// is written (the documented hazard between an M0 write and an LDS copy).
SV_DEV void copy_to_lds(const void* g, uint32_t lds_off)
{
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\t"
                 "s_mov_b32 m0, %2\n\t"
                 "s_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(g), "s"(__builtin_amdgcn_readfirstlane(lds_off))
                 : "memory");
}

// Software pipelining around the MFMAs: LDS operand reads run ahead of the
// MFMAs that use them, and register operands loaded before a loop are made
// complete before it.
#pragma once

// Makes `x` (loaded from global memory before a loop) complete here. The
// compiler's wait for such a load otherwise lands at its first use inside
// the loop, as a vmcnt(0) that each iteration would also spend waiting for
// that iteration's tile copies (issued by inline assembly the compiler does
// not count).
template <class T>
__device__ __forceinline__ void settle(T &x) {
  asm volatile("" : "+v"(x));
}

// Runs MFMA steps 0 .. N-1: step i's LDS operands, op(i), are read LA steps
// before run(i, operands) issues its MFMA. Scheduling barriers keep each
// step's reads ahead of its MFMA (without them the scheduler sinks a read to
// just before its use); the compiler then waits only for the reads a step
// uses, while the next LA steps' reads are in flight.
template <int N, int LA_, class Op, class Run>
__device__ __forceinline__ void mfma_pipelined(Op op, Run run) {
  constexpr int LA = LA_ < N ? LA_ : N;
  using T = decltype(op(0));
  T fr[LA + 1];
#pragma unroll
  for (int i = 0; i < LA; ++i) fr[i] = op(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + LA < N) fr[(i + LA) % (LA + 1)] = op(i + LA);
    __builtin_amdgcn_sched_barrier(0);
    run(i, fr[i % (LA + 1)]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

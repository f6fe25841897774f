// LDS bank probe for gfx950 (it measured 32 banks of 4 bytes, a wave64
// ds_read_b32 served as two half-waves of 32 lanes).  Each kernel below is
// one dispatch whose wave64 ds_read_b32 (or ds_read_u16) instructions follow
// one lane-address pattern;
// under rocprofv3 --pmc, SQ_LDS_BANK_CONFLICT over SQ_ACTIVE_INST_LDS per
// dispatch gives that pattern's bank-conflict cycles per LDS cycle.
//   stride<S>:        lane l reads dword l * S (the bank count shows where
//                     the conflicts start);
//   random<T, R>:     each lane reads a uniformly random entry of a table of
//                     T dwords, the bits of an entropy-coded stream being
//                     close to fair coin flips.  With R > 1 the table is
//                     held R times, laid out so that copy g occupies only
//                     banks [32 g / R, 32 (g + 1) / R) of the 32, and lane
//                     group g = (l mod 32) / (32 / R) of each half-wave
//                     reads copy g (replication with private banks);
//   random_u16<T>:    a random 2-byte entry of a table of T halfwords.
// The table holds zeros (passed in, so the compiler cannot fold them) and
// each address adds the previous value, so no load can be hoisted or merged.
// Every index is masked into the 8192-dword shared array.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kDwords = 8192;
constexpr int kIters = 1024;
constexpr uint32_t kBlocks = 2048;

__device__ __forceinline__ uint32_t xorshift(uint32_t &s) {
    s ^= s << 13;
    s ^= s >> 17;
    s ^= s << 5;
    return s;
}

__device__ __forceinline__ void fill(uint32_t *lds, uint32_t zero) {
    for (uint32_t i = threadIdx.x; i < kDwords; i += kThreads) lds[i] = zero;
    __syncthreads();
}

template <uint32_t S>
__global__ __launch_bounds__(kThreads) void stride(uint32_t *out, uint32_t zero) {
    __shared__ uint32_t lds[kDwords];
    fill(lds, zero);
    const uint32_t lane = threadIdx.x & 63u;
    uint32_t v = 0, acc = 0;
    for (int i = 0; i < kIters; i++) {
        v = lds[(lane * S + v) & (kDwords - 1)];
        acc += v;
    }
    out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <uint32_t T, uint32_t R>
__global__ __launch_bounds__(kThreads) void random(uint32_t *out, uint32_t zero) {
    constexpr uint32_t kBanks = 32, W = kBanks / R;  // banks per copy
    static_assert(T * R <= kDwords && kBanks % R == 0 && T % W == 0, "layout fits the array");
    __shared__ uint32_t lds[kDwords];
    fill(lds, zero);
    const uint32_t g = (threadIdx.x & 31u) / W;
    uint32_t s = 0x9E3779B9u * (blockIdx.x * kThreads + threadIdx.x + 1);
    uint32_t v = 0, acc = 0;
    for (int i = 0; i < kIters; i++) {
        const uint32_t e = (xorshift(s) >> 7) % T;
        const uint32_t a = R == 1 ? e : (e / W) * kBanks + g * W + e % W;
        v = lds[(a + v) & (kDwords - 1)];
        acc += v;
    }
    out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <uint32_t T>
__global__ __launch_bounds__(kThreads) void random_u16(uint32_t *out, uint32_t zero) {
    static_assert(T <= 2 * kDwords, "table fits the array");
    __shared__ uint32_t lds[kDwords];
    fill(lds, zero);
    const uint16_t *h = reinterpret_cast<const uint16_t *>(lds);
    uint32_t s = 0x85EBCA6Bu * (blockIdx.x * kThreads + threadIdx.x + 1);
    uint32_t v = 0, acc = 0;
    for (int i = 0; i < kIters; i++) {
        v = h[((xorshift(s) >> 7) % T + v) & (2 * kDwords - 1)];
        acc += v;
    }
    out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

template <class K>
int run(const char *name, K kernel, uint32_t *out) {
    hipLaunchKernelGGL(kernel, dim3(kBlocks), dim3(kThreads), 0, 0, out, 0u);
    if (hipDeviceSynchronize() != hipSuccess) {
        std::printf("%s: launch failed\n", name);
        return 1;
    }
    std::printf("%s done\n", name);
    std::fflush(stdout);
    return 0;
}

}  // namespace

int main() {
    uint32_t *out = nullptr;
    if (hipMalloc(&out, sizeof(uint32_t) * kBlocks * kThreads) != hipSuccess) return 1;
    int rc = 0;
    rc |= run("stride 1", stride<1>, out);
    rc |= run("stride 2", stride<2>, out);
    rc |= run("stride 4", stride<4>, out);
    rc |= run("stride 8", stride<8>, out);
    rc |= run("stride 16", stride<16>, out);
    rc |= run("stride 32", stride<32>, out);
    rc |= run("stride 64", stride<64>, out);
    rc |= run("stride 128", stride<128>, out);
    rc |= run("random 1024 x1", random<1024, 1>, out);
    rc |= run("random 1024 x2", random<1024, 2>, out);
    rc |= run("random 1024 x4", random<1024, 4>, out);
    rc |= run("random 1024 x8", random<1024, 8>, out);
    rc |= run("random 4096 x1", random<4096, 1>, out);
    rc |= run("random 256 x1", random<256, 1>, out);
    rc |= run("random 256 x32", random<256, 32>, out);
    rc |= run("random u16 4096", random_u16<4096>, out);
    (void)hipFree(out);
    return rc;
}

// fill.hip - GPU side of the seeded input generator: fills device-visible
// memory with the SplitMix64 byte stream and flags blocks that differ from
// it. Input generation only; no backup/restore arithmetic.
//
// Stream: word j of stream `seed` is the (j+1)-th output of SplitMix64
// (Steele, Lea and Flood, OOPSLA 2014) started at state `seed`; byte a is
// byte (a mod 8), little-endian, of word floor(a / 8).
#include <cstdint>
#include <hip/hip_runtime.h>

namespace {

__device__ __forceinline__ uint64_t word(uint64_t seed, uint64_t j)
{
    uint64_t z = seed + (j + 1) * 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

typedef uint64_t v2u64 __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(256) void fill_kernel(v2u64* out, uint64_t nvec, uint64_t seed,
                                                   uint64_t word0)
{
    for (uint64_t v = blockIdx.x * 256ull + threadIdx.x; v < nvec; v += 256ull * gridDim.x) {
        v2u64 x;
        x.x = word(seed, word0 + 2 * v);
        x.y = word(seed, word0 + 2 * v + 1);
        out[v] = x;
    }
}

__global__ __launch_bounds__(256) void diff_kernel(const v2u64* in, uint64_t nvec, uint64_t seed,
                                                   uint64_t word0, uint64_t vec_per_block,
                                                   uint32_t* flags)
{
    for (uint64_t v = blockIdx.x * 256ull + threadIdx.x; v < nvec; v += 256ull * gridDim.x) {
        const v2u64 x = in[v];
        if (x.x != word(seed, word0 + 2 * v) || x.y != word(seed, word0 + 2 * v + 1))
            flags[v / vec_per_block] = 1u;
    }
}

// device view of a pointer: pinned host memory is translated through
// hipHostGetDevicePointer, anything else is used as is
void* device_view(const void* p)
{
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, p) == hipSuccess && at.type == hipMemoryTypeHost) {
        void* d = nullptr;
        if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) == hipSuccess && d) return d;
    }
    (void)hipGetLastError();
    return const_cast<void*>(p);
}

int grid_for(uint64_t nvec)
{
    const uint64_t g = (nvec + 255) / 256;
    return static_cast<int>(g < 8192 ? (g ? g : 1) : 8192);
}

}  // namespace

extern "C" {

// Fills bytes [0, nbytes) of dev with stream bytes addr0 .. addr0+nbytes-1.
// dev 16-byte aligned, nbytes a multiple of 16, addr0 a multiple of 8.
int synth_fill(void* dev, uint64_t nbytes, uint64_t seed, uint64_t addr0, void* stream)
{
    if (!dev || (reinterpret_cast<uintptr_t>(dev) & 15) || (nbytes & 15) || (addr0 & 7)) return -1;
    if (nbytes == 0) return 0;
    const uint64_t nvec = nbytes / 16;
    hipLaunchKernelGGL(fill_kernel, dim3(grid_for(nvec)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<v2u64*>(device_view(dev)), nvec, seed,
                       addr0 / 8);
    return hipGetLastError() == hipSuccess ? 0 : -9;
}

// Sets flags[b] = 1 for every block b of block_bytes bytes of dev that holds
// a byte differing from the stream (flags must be zeroed by the caller).
int synth_diff_blocks(const void* dev, uint64_t nbytes, uint64_t seed, uint64_t addr0,
                      uint64_t block_bytes, uint32_t* flags, void* stream)
{
    if (!dev || !flags || (reinterpret_cast<uintptr_t>(dev) & 15) || (nbytes & 15) ||
        (addr0 & 7) || block_bytes == 0 || (block_bytes & 15))
        return -1;
    if (nbytes == 0) return 0;
    const uint64_t nvec = nbytes / 16;
    hipLaunchKernelGGL(diff_kernel, dim3(grid_for(nvec)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const v2u64*>(device_view(dev)), nvec,
                       seed, addr0 / 8, block_bytes / 16, flags);
    return hipGetLastError() == hipSuccess ? 0 : -9;
}

}  // extern "C"

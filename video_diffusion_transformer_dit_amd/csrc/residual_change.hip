// residual_change.hip -- Cache-DiT residual-change statistic: per sample,
// num = sum |r - r_cached|, den = sum |r_cached|, ratio = num / den over every
// token and channel of the packed sequence.
//
// Cache-DiT's reuse decision compares the boundary blocks' normalised residual
// change with the cached state (xhh.club summary of the SGLang MiniMax-H3
// benchmark, Q&A on Cache-DiT), one joint decision for the packed video+audio
// stack (stamatios.com summary, "Resultado principal").  The statistic is an
// HBM-bound read-only reduction: 4 bytes per element, nothing written but
// three doubles per sample.
//
// Determinism: stage 1 writes one fp64 (num, den) partial per 2048-vector
// tile into the caller's workspace; stage 2 reduces each sample's partials
// in a fixed order.  Every sum has a fixed shape (fp32 over the 8 values of a
// 16-byte vector, then fp64), so repeated calls give bit-identical results.
//
// The allocation-free variant keeps the partials in `scratch`, a 2 MiB array
// in the library's own device memory (one copy per GPU, held until the
// process ends).  Its device address is looked up once per device with
// hipGetSymbolAddress and cached; host code never passes the array's name
// itself to a kernel (on the host that name is only a stand-in).  Stage 1
// writes every partial stage 2 reads, so nothing in it has to start at zero.
#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"

namespace dit {

// Partials of the allocation-free entry point: B * tiles (num, den) pairs.
static __device__ __align__(256) double2 scratch[kResidualChangeScratchPartials];

namespace {

constexpr int kPartialThreads = 1024;
constexpr int kPartialU = 2; // vectors per thread per input
constexpr int kTileVectors = kPartialThreads * kPartialU;
constexpr int kFinalThreads = 1024;

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1)
        v += __shfl_xor(v, off, kWave);
    return v;
}

// grid (tiles, B).  ws[b * tiles + tile] = (num, den) of the tile.
__global__ __launch_bounds__(kPartialThreads) void residual_change_partial_kernel(const u32x4 *__restrict__ r,
                                                                                 const u32x4 *__restrict__ rc,
                                                                                 double2 *__restrict__ ws,
                                                                                 int64_t nvec, int tiles)
{
    __shared__ double2 red[kPartialThreads / kWave];
    const int tid = threadIdx.x;
    const size_t b = blockIdx.y;
    const int tile = blockIdx.x;
    const u32x4 *rs = r + b * nvec;
    const u32x4 *cs = rc + b * nvec;
    const int64_t c0 = (int64_t)tile * kTileVectors + tid;

    u32x4 va[kPartialU], vc[kPartialU];
#pragma unroll
    for (int k = 0; k < kPartialU; ++k) {
        const int64_t c = c0 + (int64_t)k * kPartialThreads;
        va[k] = vc[k] = u32x4{0u, 0u, 0u, 0u};
        if (c < nvec) {
            va[k] = load_stream(rs + c);
            vc[k] = load_stream(cs + c);
        }
    }
    double num = 0.0, den = 0.0;
#pragma unroll
    for (int k = 0; k < kPartialU; ++k) {
        float a[8], c[8];
        unpack8(va[k], a);
        unpack8(vc[k], c);
        float sn = 0.f, sd = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            sn += fabsf(a[i] - c[i]);
            sd += fabsf(c[i]);
        }
        num += (double)sn; // out-of-range vectors were zero-filled
        den += (double)sd;
    }
    num = wave_sum_f64(num);
    den = wave_sum_f64(den);
    if ((tid & (kWave - 1)) == 0)
        red[tid / kWave] = make_double2(num, den);
    __syncthreads();
    if (tid == 0) {
        double2 t = red[0];
#pragma unroll
        for (int w = 1; w < kPartialThreads / kWave; ++w) {
            t.x += red[w].x;
            t.y += red[w].y;
        }
        ws[b * tiles + tile] = t;
    }
}

// grid B.  out[3b .. 3b+2] = (num, den, ratio).
__global__ __launch_bounds__(kFinalThreads) void residual_change_final_kernel(const double2 *__restrict__ ws,
                                                                             double *__restrict__ out, int tiles)
{
    __shared__ double2 red[kFinalThreads / kWave];
    const int tid = threadIdx.x;
    const size_t b = blockIdx.x;
    double num = 0.0, den = 0.0;
    // Thread tid adds partials tid, tid + 1024, ... in that order, with eight
    // loads in flight: a single workgroup reads every partial, so latency,
    // not bandwidth, bounds this stage.
    constexpr int kInFlight = 8;
    for (int t0 = tid; t0 < tiles; t0 += kFinalThreads * kInFlight) {
        double2 p[kInFlight];
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            const int t = t0 + j * kFinalThreads;
            p[j] = t < tiles ? ws[b * tiles + t] : make_double2(0.0, 0.0);
        }
#pragma unroll
        for (int j = 0; j < kInFlight; ++j) {
            num += p[j].x;
            den += p[j].y;
        }
    }
    num = wave_sum_f64(num);
    den = wave_sum_f64(den);
    if ((tid & (kWave - 1)) == 0)
        red[tid / kWave] = make_double2(num, den);
    __syncthreads();
    if (tid == 0) {
        double2 s = red[0];
        for (int w = 1; w < kFinalThreads / kWave; ++w) {
            s.x += red[w].x;
            s.y += red[w].y;
        }
        out[3 * b + 0] = s.x;
        out[3 * b + 1] = s.y;
        out[3 * b + 2] = s.y > 0.0 ? s.x / s.y : (s.x > 0.0 ? __builtin_inf() : 0.0);
    }
}

constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mutex;
void *g_scratch_addr[kMaxScratchDevices]; // device address of `scratch`, per device id

} // namespace

hipError_t residual_change_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_addr[dev] = p;
    }
    *ptr = g_scratch_addr[dev];
    return hipSuccess;
}

int64_t residual_change_tiles(int64_t N, int64_t D) { return (N * (D / 8) + kTileVectors - 1) / kTileVectors; }

hipError_t launch_residual_change(const void *r, const void *r_cached, double *out, void *workspace, int64_t B,
                                  int64_t N, int64_t D, hipStream_t stream)
{
    const int64_t nvec = N * (D / 8);
    const int tiles = (int)residual_change_tiles(N, D);
    auto *ws = static_cast<double2 *>(workspace);
    if (tiles > 0)
        hipLaunchKernelGGL(residual_change_partial_kernel, dim3((unsigned)tiles, (unsigned)B), dim3(kPartialThreads),
                           0, stream, static_cast<const u32x4 *>(r), static_cast<const u32x4 *>(r_cached), ws, nvec,
                           tiles);
    hipLaunchKernelGGL(residual_change_final_kernel, dim3((unsigned)B), dim3(kFinalThreads), 0, stream, ws, out,
                       tiles);
    return hipGetLastError();
}

} // namespace dit

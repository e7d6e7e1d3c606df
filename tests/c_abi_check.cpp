// The C ABI used from C++ without Python: device buffers from hipMalloc, the
// calls of bitnest.h on a HIP stream, results checked against the CPU oracle
// (liboracle.so, test infrastructure). Inputs come from a counter-based
// generator (splitmix64). Checks, per problem: the activation codes and
// scales bit for bit; y within 1e-5 * max|y| of the oracle's fp64 result
// (BitNest-Llama-3-8B model card, "Files", planes.safetensors: the W4 and W8
// dequantisation); the fused quantise + linear call bit for bit equal to the
// two calls; and the host-side argument checks. Prints one line per problem
// and "c_abi_check: all passed" at the end; exits nonzero on the first
// failure.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "bitnest.h"

extern "C" {
int oracle_quant_act(const float *x, int M, int K, int act_group, int8_t *q, float *s);
int oracle_linear(int mode, const int8_t *q, const float *xs, int act_group, const uint8_t *hi, const uint8_t *lo,
                  const uint16_t *scale, int M, int N, int K, double *y64, int nthreads);
}

namespace {

int g_fail = 0;

#define CHECK(cond, ...)                                        \
    do {                                                        \
        if (!(cond)) {                                          \
            std::fprintf(stderr, "FAILED %s:%d: ", __FILE__, __LINE__); \
            std::fprintf(stderr, __VA_ARGS__);                  \
            std::fprintf(stderr, "\n");                         \
            std::exit(1);                                       \
        }                                                       \
    } while (0)

#define HIP(call)                                                                   \
    do {                                                                            \
        hipError_t e_ = (call);                                                     \
        CHECK(e_ == hipSuccess, "%s: %s", #call, hipGetErrorString(e_));            \
    } while (0)

uint64_t splitmix64(uint64_t &s) {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// uniform in [-1, 1), from the top 24 bits
float uniform(uint64_t &s) { return static_cast<float>(static_cast<int32_t>(splitmix64(s) >> 40) - (1 << 23)) / (1 << 23); }

template <typename T>
T *dev_copy(const std::vector<T> &h) {
    T *d = nullptr;
    HIP(hipMalloc(&d, h.size() * sizeof(T) + 16));
    if (!h.empty()) HIP(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

template <typename T>
std::vector<T> host_copy(const T *d, size_t n) {
    std::vector<T> h(n);
    if (n) HIP(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost));
    return h;
}

void check_status(bitnest_status st, const char *what) {
    CHECK(st == BITNEST_OK, "%s returned %d (%s)", what, static_cast<int>(st), bitnest_status_string(st));
}

void run_problem(int M, int N, int K, int act_group, bool target, uint64_t seed, hipStream_t stream) {
    const int G = K / 128, S = act_group ? G : 1;
    std::vector<float> x(static_cast<size_t>(M) * K);
    std::vector<uint8_t> hi(static_cast<size_t>(N) * K / 2), lo(hi.size());
    std::vector<uint16_t> sc(static_cast<size_t>(N) * G);
    for (auto &v : x) v = 3.0f * uniform(seed);
    x[K / 3] = 60.0f;                                            // an outlier channel
    for (auto &b : hi) b = static_cast<uint8_t>(splitmix64(seed));
    for (auto &b : lo) b = static_cast<uint8_t>(splitmix64(seed));
    for (auto &h : sc) h = static_cast<uint16_t>(0x2000 + (splitmix64(seed) % 0x0C00));   // 2^-7 .. 2^-4

    float *dx = dev_copy(x), *dy = nullptr, *dy2 = nullptr, *dxs = nullptr, *dxs2 = nullptr;
    uint8_t *dhi = dev_copy(hi), *dlo = dev_copy(lo);
    uint16_t *dsc = dev_copy(sc);
    int8_t *dxq = nullptr, *dxq2 = nullptr;
    HIP(hipMalloc(&dy, sizeof(float) * M * N + 16));
    HIP(hipMalloc(&dy2, sizeof(float) * M * N + 16));
    HIP(hipMalloc(&dxs, sizeof(float) * M * S + 16));
    HIP(hipMalloc(&dxs2, sizeof(float) * M * S + 16));
    HIP(hipMalloc(&dxq, static_cast<size_t>(M) * K + 16));
    HIP(hipMalloc(&dxq2, static_cast<size_t>(M) * K + 16));

    // two calls, then the fused call on separate outputs
    check_status(bitnest_quant_act(dx, M, K, act_group, dxq, dxs, stream), "bitnest_quant_act");
    if (target) {
        check_status(bitnest_linear_target(dxq, dxs, act_group, dhi, dlo, dsc, dy, M, N, K, stream),
                     "bitnest_linear_target");
        check_status(bitnest_quant_linear_target(dx, act_group, dhi, dlo, dsc, dy2, dxq2, dxs2, M, N, K, stream),
                     "bitnest_quant_linear_target");
    } else {
        check_status(bitnest_linear_draft(dxq, dxs, act_group, dhi, dsc, dy, M, N, K, stream), "bitnest_linear_draft");
        check_status(bitnest_quant_linear_draft(dx, act_group, dhi, dsc, dy2, dxq2, dxs2, M, N, K, stream),
                     "bitnest_quant_linear_draft");
    }
    HIP(hipStreamSynchronize(stream));
    const auto q = host_copy(dxq, static_cast<size_t>(M) * K), q2 = host_copy(dxq2, static_cast<size_t>(M) * K);
    const auto s = host_copy(dxs, static_cast<size_t>(M) * S), s2 = host_copy(dxs2, static_cast<size_t>(M) * S);
    const auto y = host_copy(dy, static_cast<size_t>(M) * N), y2 = host_copy(dy2, static_cast<size_t>(M) * N);

    std::vector<int8_t> q_ref(q.size());
    std::vector<float> s_ref(s.size());
    CHECK(oracle_quant_act(x.data(), M, K, act_group, q_ref.data(), s_ref.data()) == 0, "oracle_quant_act");
    CHECK(std::memcmp(q.data(), q_ref.data(), q.size()) == 0, "codes differ from the oracle");
    CHECK(std::memcmp(s.data(), s_ref.data(), s.size() * sizeof(float)) == 0, "scales differ from the oracle");
    CHECK(std::memcmp(q.data(), q2.data(), q.size()) == 0, "fused codes differ from the two calls");
    CHECK(std::memcmp(s.data(), s2.data(), s.size() * sizeof(float)) == 0, "fused scales differ");
    CHECK(std::memcmp(y.data(), y2.data(), y.size() * sizeof(float)) == 0, "fused y differs from the two calls");

    std::vector<double> y64(static_cast<size_t>(M) * N);
    CHECK(oracle_linear(target ? 1 : 0, q_ref.data(), s_ref.data(), act_group, hi.data(), target ? lo.data() : nullptr,
                        sc.data(), M, N, K, y64.data(), 0) == 0, "oracle_linear");
    double ref = 0.0, err = 0.0;
    for (size_t i = 0; i < y64.size(); ++i) {
        ref = std::fmax(ref, std::fabs(y64[i]));
        err = std::fmax(err, std::fabs(static_cast<double>(y[i]) - y64[i]));
    }
    CHECK(err <= 1e-5 * ref, "y: max error %.3e against the bound %.3e", err, 1e-5 * ref);
    std::printf("M=%d N=%d K=%d act_group=%d %s: codes, scales exact; max|y - oracle| = %.3e (bound %.3e)\n", M, N,
                K, act_group, target ? "target" : "draft", err, 1e-5 * ref);

    for (void *p : {static_cast<void *>(dx), static_cast<void *>(dy), static_cast<void *>(dy2),
                    static_cast<void *>(dxs), static_cast<void *>(dxs2), static_cast<void *>(dhi),
                    static_cast<void *>(dlo), static_cast<void *>(dsc), static_cast<void *>(dxq),
                    static_cast<void *>(dxq2)})
        HIP(hipFree(p));
}

void check_argument_errors(hipStream_t stream) {
    // refused on the host before any launch
    float *d = nullptr;
    HIP(hipMalloc(&d, 1 << 20));
    auto *b = reinterpret_cast<uint8_t *>(d);
    auto *q = reinterpret_cast<int8_t *>(d);
    auto *h = reinterpret_cast<uint16_t *>(d);
    CHECK(bitnest_linear_draft(q, d, 0, b, h, d, 1, 16, 100, stream) == BITNEST_EINVAL, "K not a multiple of 128");
    CHECK(bitnest_linear_draft(q, d, 64, b, h, d, 1, 16, 128, stream) == BITNEST_EINVAL, "act_group 64");
    CHECK(bitnest_linear_draft(q, d, 0, b + 1, h, d, 1, 16, 128, stream) == BITNEST_EALIGN, "misaligned plane");
    CHECK(bitnest_linear_draft(q, d, 0, b, h, d, BITNEST_MAX_M + 1, 16, 128, stream) == BITNEST_EUNSUPPORTED,
          "M above the maximum");
    CHECK(bitnest_linear_target(q, d, 0, b, nullptr, h, d, 1, 16, 128, stream) == BITNEST_EINVAL, "target without lo");
    CHECK(bitnest_linear_draft(nullptr, nullptr, 0, nullptr, nullptr, nullptr, 0, 16, 128, stream) == BITNEST_OK,
          "M = 0 is a no-op");
    CHECK(std::strlen(bitnest_status_string(BITNEST_EALIGN)) > 0, "status string");
    CHECK(bitnest_abi_version() == BITNEST_ABI_VERSION, "ABI version %d, header %d", bitnest_abi_version(),
          BITNEST_ABI_VERSION);
    HIP(hipFree(d));
    std::printf("argument checks: ok\n");
}

}  // namespace

int main() {
    int n = 0;
    HIP(hipGetDeviceCount(&n));
    CHECK(n > 0, "no HIP device");
    HIP(hipSetDevice(0));
    hipStream_t stream;
    HIP(hipStreamCreate(&stream));
    check_argument_errors(stream);
    struct Problem { int M, N, K, g; bool target; };
    const Problem problems[] = {
        {1, 256, 512, 0, false}, {1, 256, 512, 0, true}, {1, 1000, 4096, 128, false}, {4, 300, 4096, 0, true},
        {4, 77, 14336, 0, true}, {3, 129, 2176, 128, false}, {8, 200, 4096, 0, true}, {32, 64, 1024, 128, false},
        {2, 5, 16384, 0, true},
    };
    uint64_t seed = 0x5EED;
    for (const auto &p : problems) run_problem(p.M, p.N, p.K, p.g, p.target, seed++, stream);
    HIP(hipStreamDestroy(stream));
    std::printf("c_abi_check: all passed\n");
    return g_fail;
}

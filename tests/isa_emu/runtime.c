/* A stand-in for the HIP runtime, for running the library's host code on the
 * CPU: it registers kernels and device variables as the real runtime would,
 * and hands every kernel launch (name, grid, block, argument pointers) to a
 * callback, the instruction-level emulator.  Device memory is process memory.
 * Only the entry points the library imports are provided; the version node
 * matches the one the library was linked against. */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <stdio.h>

typedef struct { uint32_t x, y, z; } dim3;
typedef int hipError_t;

typedef int (*launch_cb_t)(const char* name, uint32_t gx, uint32_t gy, uint32_t gz,
                           uint32_t bx, uint32_t by, uint32_t bz, size_t shmem,
                           void** args, void* stream);
static launch_cb_t g_cb = 0;
static int g_cu_count = 8;
static int g_last_err = 0;

#define MAXF 256
static const void* f_host[MAXF];
static const char* f_name[MAXF];
static int n_f = 0;

#define MAXV 64
static void* v_host[MAXV];
static const char* v_name[MAXV];
static size_t v_size[MAXV];
static void* v_dev[MAXV];
static int n_v = 0;

static dim3 cfg_grid[16], cfg_block[16];
static size_t cfg_shmem[16];
static void* cfg_stream[16];
static int n_cfg = 0;

void emu_set_launch_callback(launch_cb_t cb) { g_cb = cb; }
void emu_set_cu_count(int n) { g_cu_count = n; }
int emu_var_count(void) { return n_v; }
void emu_var_info(int i, const char** name, void** dev, size_t* size) {
  *name = v_name[i]; *dev = v_dev[i]; *size = v_size[i];
}

void** __hipRegisterFatBinary(const void* data) { (void)data; static void* h[4]; return h; }
void __hipUnregisterFatBinary(void** m) { (void)m; }
void __hipRegisterFunction(void** modules, const void* hostFunction, char* deviceFunction,
                           const char* deviceName, unsigned int threadLimit, void* tid,
                           void* bid, void* blockDim, void* gridDim, int* wSize) {
  (void)modules; (void)deviceFunction; (void)threadLimit; (void)tid; (void)bid;
  (void)blockDim; (void)gridDim; (void)wSize;
  if (n_f < MAXF) { f_host[n_f] = hostFunction; f_name[n_f] = deviceName; n_f++; }
}
void __hipRegisterVar(void** modules, void* var, char* hostVar, char* deviceVar, int ext,
                      size_t size, int constant, int global) {
  (void)modules; (void)hostVar; (void)ext; (void)constant; (void)global;
  if (n_v < MAXV) { v_host[n_v] = var; v_name[n_v] = deviceVar; v_size[n_v] = size; v_dev[n_v] = 0; n_v++; }
}
hipError_t __hipPushCallConfiguration(dim3 g, dim3 b, size_t shmem, void* stream) {
  if (n_cfg >= 16) return 1;
  cfg_grid[n_cfg] = g; cfg_block[n_cfg] = b; cfg_shmem[n_cfg] = shmem; cfg_stream[n_cfg] = stream;
  n_cfg++;
  return 0;
}
hipError_t __hipPopCallConfiguration(dim3* g, dim3* b, size_t* shmem, void** stream) {
  if (n_cfg <= 0) return 1;
  n_cfg--;
  *g = cfg_grid[n_cfg]; *b = cfg_block[n_cfg]; *shmem = cfg_shmem[n_cfg]; *stream = cfg_stream[n_cfg];
  return 0;
}
hipError_t hipLaunchKernel(const void* f, dim3 g, dim3 b, void** args, size_t shmem, void* stream) {
  for (int i = 0; i < n_f; i++)
    if (f_host[i] == f) {
      if (!g_cb) { fprintf(stderr, "fakehip: no launch callback\n"); abort(); }
      int r = g_cb(f_name[i], g.x, g.y, g.z, b.x, b.y, b.z, shmem, args, stream);
      if (r) { g_last_err = 98; return 98; }
      return 0;
    }
  fprintf(stderr, "fakehip: launch of an unregistered function\n");
  abort();
}
/* the timed launch of the measurement hook: events are not modelled */
hipError_t hipExtLaunchKernel(const void* f, dim3 g, dim3 b, void** args, size_t shmem,
                              void* stream, void* start, void* stop, int flags) {
  (void)start; (void)stop; (void)flags;
  return hipLaunchKernel(f, g, b, args, shmem, stream);
}
hipError_t hipGetLastError(void) { int e = g_last_err; g_last_err = 0; return e; }
const char* hipGetErrorString(hipError_t e) { return e ? "emulated launch failed" : "no error"; }
hipError_t hipGetDevice(int* d) { *d = 0; return 0; }
hipError_t hipDeviceGetAttribute(int* v, int attr, int dev) {
  (void)dev;
  /* hipDeviceAttributeMultiprocessorCount and anything else: the CU count */
  (void)attr; *v = g_cu_count; return 0;
}
hipError_t hipEventCreate(void** e) { static int dummy; *e = &dummy; return 0; }
hipError_t hipEventRecord(void* e, void* s) { (void)e; (void)s; return 0; }
hipError_t hipEventSynchronize(void* e) { (void)e; return 0; }
hipError_t hipEventElapsedTime(float* ms, void* a, void* b) { (void)a; (void)b; *ms = 0.f; return 0; }
hipError_t hipGetSymbolAddress(void** p, const void* sym) {
  for (int i = 0; i < n_v; i++)
    if (v_host[i] == sym) {
      if (!v_dev[i]) { v_dev[i] = aligned_alloc(4096, (v_size[i] + 4095) & ~(size_t)4095);
                       memset(v_dev[i], 0xA5, v_size[i]); }
      *p = v_dev[i];
      return 0;
    }
  return 13;
}

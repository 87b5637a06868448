/* Module-registration hooks for a host-only build of libgq (device code
 * compiled out): the compiler's module constructors call these with the
 * device-code images and kernel names.  Defined in the test executable, they
 * take precedence over the HIP runtime's and do nothing, so the runtime never
 * sees the empty images.  No kernel is launched by the host checks. */
#include <stddef.h>

static void *g_handle;

void **__hipRegisterFatBinary(const void *data) {
  (void)data;
  return &g_handle;
}
void __hipUnregisterFatBinary(void **modules) { (void)modules; }
void __hipRegisterFunction(void **modules, const void *host_fn, char *dev_fn, const char *dev_name,
                           unsigned int thread_limit, void *tid, void *bid, void *block_dim,
                           void *grid_dim, int *wsize) {
  (void)modules; (void)host_fn; (void)dev_fn; (void)dev_name; (void)thread_limit;
  (void)tid; (void)bid; (void)block_dim; (void)grid_dim; (void)wsize;
}
void __hipRegisterVar(void **modules, void *var, char *host_var, char *dev_var, int ext, size_t size,
                      int constant, int global) {
  (void)modules; (void)var; (void)host_var; (void)dev_var; (void)ext; (void)size; (void)constant;
  (void)global;
}
